// Internal interface between the C-ABI front end (mgqa_api.cpp) and the
// gfx950 kernels (mgqa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mgqa {

// Prefill kernels: 8 waves x 2 blocks of 16 rows, every wave sweeps whole
// 64-key tiles.
constexpr int kPrefillKeys = 64;
constexpr int kPrefillWaves = 8;
constexpr int kPrefillNqb = 2;
// Head sizes 104-120 (four 32-wide Q chunks, 128-wide P.V): one block of 16
// rows per wave; with two, the accumulators and the staged next tile need
// more than the 256 registers an 8-wave workgroup allows and spill.
constexpr int kPrefillNqbWide = 1;
// Head size 128: four waves x 2 blocks of 16 rows, 32-key tiles.
constexpr int kPipe4Waves = 4;
constexpr int kPipe4Keys = 32;
// Split-KV kernel: waves per workgroup; each wave takes 32 keys of a tile.
constexpr int kSplitWaves = 4;
constexpr int kSplitKeys = 32 * kSplitWaves;
// Wide split workgroups: 8 waves over 256-key tiles, for one 16-row block with
// a long key range per workgroup (decode).
constexpr int kSplitWavesWide = 8;
constexpr int kSplitWideMinTiles = 8;  // 128-key tiles per workgroup from which they are used
constexpr int kSplitMaxNqb = 4;     // 16-row blocks per workgroup, head size <= 96
constexpr int kSplitMaxNqbWide = 2; // head size > 96 (register budget)
constexpr int kSplitWideMaxDv = 6;  // P.V 16-column blocks up to which 3 and 4 row blocks exist

// Short-band kernel (encoder-sized sequences): 8 waves x three 16-row
// blocks per workgroup; each wave takes up to three 32-key steps of the
// block's key band, so a band of at most 24 steps (768 keys) fits.
constexpr int kEncWaves = 8;
constexpr int kEncSteps = 3;
constexpr int kEncNqb = 3;
constexpr int kEncMaxSteps = kEncWaves * kEncSteps;

enum Path { kPathPrefill = 0, kPathSplit = 1, kPathShort = 2 };

// Division by a launch constant without a divide sequence: for 0 <= x < 2^31,
// x / d == (x * m) >> (31 + s) with s = ceil(log2 d) and m = ceil(2^(31+s) / d)
// (m < 2^32; the rounding error x*(m - 2^(31+s)/d) / 2^(31+s) stays below 2^-s
// <= 1/d, so it never carries past an integer).
struct FastDiv {
  uint32_t m;
  uint32_t s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1u << s) < d) ++s;
  const uint64_t num = 1ull << (31 + s);
  return FastDiv{(uint32_t)((num + d - 1) / d), s};
}

// Everything a kernel needs, passed by value.
struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* ws_o;        // split partial outputs [group][split][nrows][dv_pad]
  float* ws_ml;       // split partial (max, sum) [group][split][nrows][2]
  unsigned* ws_cnt;   // split arrival counters [group]; group = unit * n_pos_blk + position block
  int Hq, Hkv, G, Lq, Lkv, d;
  long long kv_stride;  // elements between consecutive (batch, kv head) units of K and V
  int ring_start;       // -1: linear keys; else key j lives in slot (ring_start + j) % ring_slots
  int ring_slots;
  int causal, window;
  float alpha;        // log2(e)/sqrt(d): raw score -> base-2 exponent units
  float gamma;        // 2*log2(e)/(c*sqrt(d)): softcap exp argument
  float c2;           // c*log2(e): softcapped score bound in exponent units
  float beta;         // 1/(c*sqrt(d))
  int m;              // query positions per workgroup
  int n_pos_blk;      // position blocks per (batch, kv head)
  // split path
  int nsplit;         // key splits per position block
  int tiles_per_split;
  int nrows;          // m*G rows of a full position block
  FastDiv div_g, div_hkv, div_npos, div_nsplit;  // for G, Hkv, n_pos_blk, nsplit
  int nwg;            // workgroups of the launch (the grid size, read with the other arguments)
  // Fused cache append (split path, linear cache): keys app_pos .. app_pos+app_len-1
  // (one per query position) come from the float32 rows app_k / app_v
  // ([unit][app_len][d]) and are written to K / V.  app_len 0: no append.
  const float* app_k;
  const float* app_v;
  int app_pos, app_len;
  // Pipelined head-size-128 prefill: pf_items work items per unit -- pf_pairs
  // pairs of the first pf_ramp position blocks, pf_full whole blocks, then
  // half blocks (two items each).
  int pf_items, pf_pairs, pf_ramp, pf_full;
  FastDiv div_items;  // for pf_items
};

struct Plan {
  int path;
  int dqk;            // 32-wide head-size steps for Q.K^T
  int qk_pad;         // head size Q.K^T is contracted over (padded)
  int dv;             // 16-wide head-size blocks for P.V
  int nqb;            // 16-row query blocks per wave
  int nwaves;         // waves per workgroup
  int rows_per_wg;
  int keys_per_tile;
  int m;              // query positions per workgroup
  int n_pos_blk;      // position blocks per (batch, kv head)
  int nsplit;
  int tiles_per_split;
  int ncol;           // split path: workgroups sharing one key range, each with 1/ncol of V's columns
  int pf_items, pf_pairs, pf_ramp, pf_full;  // pipelined prefill work items (see KernelArgs)
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
