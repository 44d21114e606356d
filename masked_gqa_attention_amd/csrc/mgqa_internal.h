// Internal interface between the C-ABI front end (mgqa_api.cpp) and the
// gfx950 kernels (mgqa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mgqa {

// Keys per staged tile.
constexpr int kPrefillKeys = 64;   // prefill/encoder: every wave sweeps the whole tile
#ifndef MGQA_DECODE_WAVES
#define MGQA_DECODE_WAVES 8
#endif
constexpr int kDecodeWaves = MGQA_DECODE_WAVES;  // split decode: waves per workgroup
constexpr int kDecodeKeys = 32 * kDecodeWaves;    // each wave takes 32 keys of a tile
constexpr int kThreads = 256;      // 4 wave64 per workgroup
constexpr int kMaxRowsDecode = 16; // one 16-column MFMA block of (head, position) rows

enum Path { kPathPrefill = 0, kPathDecode = 1 };

// Everything a kernel needs, passed by value.
struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* ws_o;        // decode partial outputs [unit][split][nrows][dv_pad]
  float* ws_ml;       // decode partial (max, sum) [unit][split][nrows][2]
  unsigned* ws_cnt;   // decode arrival counters [unit]
  int Hq, Hkv, G, Lq, Lkv, d;
  long long kv_stride;  // elements between consecutive (batch, kv head) units of K and V
  int ring_start;       // -1: linear keys; else key j lives in slot (ring_start + j) % ring_slots
  int ring_slots;
  int causal, window;
  float alpha;        // log2(e)/sqrt(d): raw score -> base-2 exponent units
  float gamma;        // 2*log2(e)/(c*sqrt(d)): softcap exp argument
  float c2;           // c*log2(e): softcapped score bound in exponent units
  float beta;         // 1/(c*sqrt(d))
  // prefill
  int m;              // query positions per workgroup
  int n_pos_blk;      // position blocks per (batch, kv head)
  // decode
  int nsplit;         // splits per unit
  int tiles_per_split;
  int t_begin;        // first key tile of the band (same for every unit)
  int t_end;          // one past the last key tile
  int nrows;          // G*Lq rows per unit
};

struct Plan {
  int path;
  int dqk;            // 32-wide head-size steps for Q.K^T
  int dv;             // 16-wide head-size blocks for P.V
  int nqb;            // prefill: 16-row query blocks per wave
  int nwaves;         // prefill: waves per workgroup
  int rows_per_wg;
  int keys_per_tile;
  int nsplit;
  int tiles_per_split;
  long long workgroups;
  size_t ws_bytes;
  size_t ws_o_off, ws_ml_off, ws_cnt_off;
};

// Returns 0 and fills the plan, or a negative MGQA_ERR_* code.
int make_plan(int B, int Hq, int Hkv, int Lq, int Lkv, int d, int causal, int window,
              float softcap, int dtype, Plan* plan);

// Launches the planned kernels on `stream`.  Returns a hipError_t value.
int launch(const Plan& plan, const KernelArgs& args, int dtype, bool softcap, void* stream);

// Zero-fills `words` 32-bit words at `p` with a kernel on `stream`.
int launch_zero(void* p, size_t words, void* stream);

// KV-cache append (arguments validated by the caller).  Returns a hipError_t.
int launch_append(void* kc, void* vc, const float* nk, const float* nv, int B, int S, int H, int D,
                  int L, int position, int cache_dtype, int layout, int* length_out, void* stream);

}  // namespace mgqa
