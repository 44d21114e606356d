// gfx950 (MI355X, CDNA4) kernels for masked grouped-query attention.
//
// Operation: the attention forward pass of the task page "TPU v6e Masked GQA
// Kernel Optimization" ("What You Have": decode, prefill and encoder shapes,
// GQA 1:1 to 16:1, optional causal mask, sliding window and logit softcap).
// The score/probability products run on bf16/fp16 MFMA with fp32 accumulation
// (the Graphcore page, "SigLIP batch-1 hardware results", uses the same split of
// 16-bit products and 32-bit accumulation); the softmax is fp32 and streams
// over key tiles (the "bounded-block" streaming form named on that page's
// introduction), so the score matrix is never materialised.
//
// Layout of the work:
//   * A workgroup owns one (batch, kv head) pair and a block of query rows.  A
//     row is a (query head of the group, query position) pair, so one K/V tile
//     staged in LDS feeds all G query heads that share the kv head.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32:
//     the accumulator layout of S^T (lane = query column, 4 consecutive keys
//     per lane group and 16-key block) is the B-operand layout P^T needs for
//     the second product O^T = V^T P^T, so probabilities never leave
//     registers.  The V^T operand comes from row-major V in LDS through the
//     transposing LDS read ds_read_b64_tr_b16.
//   * K and V tiles are staged row-major: through registers with buffer loads
//     (padded rows), or -- head size 128 -- straight from HBM into LDS with
//     buffer loads that write LDS (dense rows, swizzled 16-byte slots).  Keys
//     past the end fall outside the buffer range and read as zero.
//   * Tiles wholly outside the causal/window band are never visited; tiles
//     wholly inside skip the mask arithmetic.
//   * Online softmax in base 2 with a lazily updated reference maximum: the
//     accumulators are rescaled only when a row maximum grows by more than
//     2^8, so probabilities stay below 256 and most steps skip the rescale.
//   * Decode (G*Lq <= 16 rows per kv head) splits the key band over
//     workgroups; each writes fp32 partials (max, sum, unnormalised output) and
//     the last workgroup to arrive for a (batch, kv head) combines all splits in
//     split order.  No float atomics: the result is bit-reproducible.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mgqa_internal.h"
#ifdef MGQA_TIMELINE
#include "mgqa.h"
#include "mgqa_timeline.h"
#endif

namespace mgqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
// Lazy rescale threshold in base-2 exponent units.
constexpr float kRescaleSlack = 8.0f;

// ---------------------------------------------------------------------------
// Timeline build (compiled with MGQA_TIMELINE defined; in the library proper
// every Timeline call below is an empty inline function and generates no
// code).  At each event of its kernel a wave reads the 100 MHz real-time
// counter, between scheduling barriers so that the compiler moves no work
// across the mark, and keeps it in one lane of a single vector register
// (lanes 0-7: low words of events 0-7, lanes 8-15: high words, lane 16: the
// record slot), so that a mark holds no scalar registers and issues no
// memory operation.  When the wave ends, lanes 0-17 write the record.  Record
// layout and the events of each kernel: include/mgqa_timeline.h.
// ---------------------------------------------------------------------------
#ifdef MGQA_TIMELINE
constexpr int kTlEvents = MGQA_TIMELINE_EVENTS;
constexpr int kTlMaxWaves = MGQA_TIMELINE_MAX_WAVES;
static_assert(kTlEvents == 8, "lanes 0-15 hold the event times");
__device__ __attribute__((aligned(256))) unsigned long long g_timeline[(size_t)kTlMaxWaves * (kTlEvents + 1)];

struct Timeline {
  unsigned v;
  // Lane LANE of v = x (x wave-uniform).
  template <int LANE>
  __device__ __forceinline__ void put(unsigned x) {
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(x), "i"(LANE));
  }
  __device__ __forceinline__ explicit Timeline(int waves) {
    v = 0u;
    put<16>(__builtin_amdgcn_readfirstlane(blockIdx.x * (unsigned)waves + (threadIdx.x >> 6)));
  }
  template <int EV>
  __device__ __forceinline__ void mark() {
    static_assert(EV >= 0 && EV < kTlEvents, "event index");
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long t = __builtin_amdgcn_s_memrealtime();
    put<EV>((unsigned)t);
    put<8 + EV>((unsigned)(t >> 32));
    __builtin_amdgcn_sched_barrier(0);
  }
  // Word 0 = 1 | XCD << 4 | HW_ID << 32; events not reached read 0.
  __device__ __forceinline__ void flush() {
    const unsigned slot = __builtin_amdgcn_readlane(v, 16);
    if (slot >= (unsigned)kTlMaxWaves) return;
    unsigned xcc, hw;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    unsigned* rec = reinterpret_cast<unsigned*>(g_timeline + (size_t)slot * (kTlEvents + 1));
    const int lane = threadIdx.x & 63;
    if (lane < 16)
      rec[2 + 2 * (lane & 7) + (lane >> 3)] = v;
    else if (lane == 16)
      rec[0] = 1u | ((xcc & 0xFu) << 4);
    else if (lane == 17)
      rec[1] = hw;
  }
};
#else
struct Timeline {
  __device__ __forceinline__ explicit Timeline(int) {}
  template <int EV>
  __device__ __forceinline__ void mark() {}
  __device__ __forceinline__ void flush() {}
};
#endif

// ---------------------------------------------------------------------------
// Element-type traits: the MFMA and the float -> storage conversion.
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
  }
};

template <>
struct Elem<_Float16> {
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 f = {lo, hi};
    f16x2 h = __builtin_convertvector(f, f16x2);
    return __builtin_bit_cast(uint32_t, h);
  }
};

// All-ones matrix-core operand (two 16-bit 1.0 per dword): multiplying it by
// P^T gives the row sums of P in every row of the result.
template <typename T>
struct OnesOperand;
template <>
struct OnesOperand<__bf16> {
  static constexpr uint32_t kPair = 0x3F803F80u;  // two bf16 1.0
};
template <>
struct OnesOperand<_Float16> {
  static constexpr uint32_t kPair = 0x3C003C00u;  // two fp16 1.0
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Split partials cross workgroups (and XCDs, each with its own L2) through
// device-scope stores and loads, which write through to and read from the
// device coherence point.  The writer waits for its stores to
// complete before it bumps the arrival counter, so the last arrival reads
// complete partials.  This avoids device-scope fences, which on this chip
// write back and invalidate the whole L2 of the XCD.
// Buffer instructions carry the scope bits: kDeviceScope sets SC1 (device
// scope, SC0 clear).  The descriptor's third dword is the gfx9 raw-buffer
// format word (32-bit data format, no swizzle).
constexpr int kDeviceScope = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st_dev16(__amdgpu_buffer_rsrc_t rs, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kDeviceScope);
}
__device__ __forceinline__ void st_dev8(__amdgpu_buffer_rsrc_t rs, int off, f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, off, 0, kDeviceScope);
}
__device__ __forceinline__ f32x4 ld_dev16(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kDeviceScope));
}
__device__ __forceinline__ f32x2 ld_dev8(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kDeviceScope));
}
// Wait until every vector-memory operation this wave issued has completed
// (s_waitcnt vmcnt(0); the expcnt and lgkmcnt fields are left at "no wait").
__device__ __forceinline__ void wait_vmem_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Butterfly steps across the four 16-lane groups of a wave (the lanes that
// hold one MFMA column).  v_permlane16_swap / v_permlane32_swap applied to a
// value and a copy of it leave, in each lane, the value and that of lane ^ 16
// (lane ^ 32) in the two registers; the max or sum of the pair is the
// butterfly step, with no LDS round trip.  The sum is the same in both lanes of
// a pair.  (The two results are copied out as integers before the bit cast:
// a bit cast applied directly to an element of the returned vector reads the
// first element for both.)
template <bool X32>
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  unsigned r0, r1;
  if constexpr (X32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
// (A compare and select: no NaN quieting of the bit-cast values needed.)
__device__ __forceinline__ float xor16_max(float x) {
  float a, b;
  lane_pair<false>(x, a, b);
  return a > b ? a : b;
}
__device__ __forceinline__ float xor32_max(float x) {
  float a, b;
  lane_pair<true>(x, a, b);
  return a > b ? a : b;
}
__device__ __forceinline__ float xor16_sum(float x) {
  float a, b;
  lane_pair<false>(x, a, b);
  return a + b;
}
__device__ __forceinline__ float xor32_sum(float x) {
  float a, b;
  lane_pair<true>(x, a, b);
  return a + b;
}
// Max / sum over the four lanes l % 16 == c of a column.
__device__ __forceinline__ float col_max(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float col_sum(float x) { return xor32_sum(xor16_sum(x)); }

// Visibility of global key `j` to a row at absolute key position `pos`.
__device__ __forceinline__ bool key_visible(int j, int pos, int Lkv, int causal, int window) {
  bool ok = j < Lkv;
  if (causal) ok = ok && (j <= pos);
  if (window > 0) {
    ok = ok && (pos - j < window);
    if (!causal) ok = ok && (j - pos < window);
  }
  return ok;
}

// Load this lane's Q^T operand (16 query columns, 8 head-size elements per
// lane group and 32-wide step).  Rows outside the problem load zeros.
template <int DQK>
__device__ __forceinline__ void load_q(u32x4 (&qf)[DQK], const uint16_t* qrow, bool ok, int d,
                                       int g4) {
#pragma unroll
  for (int t = 0; t < DQK; ++t) {
    const int col = 32 * t + 8 * g4;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (ok && col < d) val = ldg16(qrow + col);
    qf[t] = val;
  }
}

// Store one lane's 16-row x (DV*16) output slice: lane column c16 is the row,
// lane group g4 holds head-size columns 16*db + 4*g4 + [0..3].
template <typename T, int DV>
__device__ __forceinline__ void store_row(uint16_t* orow, const f32x4 (&o)[DV], float inv, int d,
                                          int g4) {
#pragma unroll
  for (int db = 0; db < DV; ++db) {
    const int col = 16 * db + 4 * g4;
    if (col < d) {
      u32x2 w = {Elem<T>::pack2(o[db][0] * inv, o[db][1] * inv),
                 Elem<T>::pack2(o[db][2] * inv, o[db][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + col) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill path.  K and V tiles are both staged row-major ([key][head size],
// rows padded); V is read transposed straight from LDS with
// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element j%4
// of the 8-byte rows addressed by lanes 4e + j/4 (e = 0..3).  Pointing lane s
// at row key0 + s/4, columns c0 + 4*(s%4) .. +3 therefore hands lane j the
// four keys key0..key0+3 of column c0 + j: the A-operand slice of V^T.
// ---------------------------------------------------------------------------

// Row-major tile [KEYS][PITCH] of 16-bit elements moved by NT threads in
// 16-byte chunks, CH chunks per row.  Loads are raw buffer loads through a
// descriptor based at the tile's first key whose range ends at Lkv, so keys
// past Lkv read as zero in hardware; chunks past d get an offset beyond any
// range and read as zero too.  Per-thread offsets are loop invariant.
//
// Offsets are unsigned 32-bit bytes.  The front end keeps every (batch, kv
// head) unit at most 2^30 elements (2^31 bytes), so kOutOfRange, even plus the
// row steps of a tile, is never inside a descriptor's range.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Cache policy of a buffer load: 0, or kStreamLoad, the non-temporal bit
// (the lines are kept in the caches only briefly).  The split-KV kernel
// reads K/V with it when every (unit, split) key range is read by one
// workgroup, or by the two column halves of a range at the same time: one
// position block per unit, as in decode.  Measured against plain loads, same
// box, median of 30 rounds: decode 4:1 over 8192 keys 47.0 -> 44.1 us, the
// long windowed decode 13.4 -> 12.75 us, 4:1 over 2048 keys 16.6 -> 15.1 us.
// With several position blocks re-reading a unit's rows through L2 it costs
// those hits (300 queries over 4096 keys, 16 heads: 70 -> 103 us), so those
// plans keep plain loads.
constexpr int kStreamLoad = 2;

template <int KEYS, int CH, int PITCH, int NT, int AUX = 0>
struct RowTile {
  static constexpr int TOTAL = KEYS * CH;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  // When NT is a multiple of CH every load of a thread has the same column
  // chunk, so one base offset and a uniform row step describe all of them.
  static constexpr bool COMPACT = (NT % CH == 0) && (TOTAL % NT == 0);
  static constexpr int NOFF = COMPACT ? 1 : PER;
  u32x4 r[PER];
  uint32_t voff[NOFF];
  uint32_t vstep;  // bytes between consecutive loads of a thread (COMPACT only)

  // col0: first column of the rows this tile holds (a multiple of 8).
  __device__ __forceinline__ void init(int d, int tid, int col0 = 0) {
    vstep = (uint32_t)((NT / CH) * d * 2);
#pragma unroll
    for (int it = 0; it < NOFF; ++it) {
      const int c = tid + it * NT;
      const int key = c / CH, ch = c % CH;
      const bool ok = (TOTAL % NT == 0 || c < TOTAL) && (col0 + ch * 8 < d);
      voff[it] = ok ? (uint32_t)((key * d + col0 + ch * 8) * 2) : kOutOfRange;
    }
  }
  // g: the (batch, kv head) unit's first row; loads keys k0 .. k0+KEYS-1.
  __device__ __forceinline__ void load(const uint16_t* g, int k0, int Lkv, int d) {
    const auto rs = make_rsrc(g + (size_t)k0 * d, (uint32_t)(Lkv - k0) * (uint32_t)d * 2u);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const uint32_t vo = COMPACT ? voff[0] + (uint32_t)it * vstep : voff[it];
      r[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)vo, 0, AUX));
    }
  }
  // Ring-buffer cache: logical key j of the unit lives in slot
  // (ring_start + j) % S; logical keys at or past Lkv, and chunks past d, read
  // as zero (offset beyond the unit's range).  g: the unit's slot 0.
  __device__ __forceinline__ void load_ring(const uint16_t* g, int k0, int Lkv, int d, int ring_start,
                                            int S, int tid, int col0 = 0) {
    const auto rs = make_rsrc(g, (uint32_t)S * (uint32_t)d * 2u);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = tid + it * NT;
      const int logical = k0 + c / CH, ch = c % CH;
      int slot = ring_start + logical;
      slot -= (slot >= S) ? S : 0;
      const bool ok = (TOTAL % NT == 0 || c < TOTAL) && (logical < Lkv) && (col0 + ch * 8 < d);
      const uint32_t vo = ok ? (uint32_t)(slot * d + col0 + ch * 8) * 2u : kOutOfRange;
      r[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)vo, 0, AUX));
    }
  }
  // Fused cache append: the chunks of keys app_pos .. app_pos+app_len-1 of the
  // tile at k0 take the float32 rows src ([app_len][d]) rounded to T (nearest
  // even) instead of what load() / load_ring() fetched; the chunks of the keys
  // whose index minus app_pos lies in [wlo, whi) are also stored to their
  // cache slot at dst (the unit's slot 0; nullptr: no stores): slot j, or
  // (ring_start + j) mod S for a ring.  Runs only for tiles that hold appended
  // keys.
  template <typename T>
  __device__ __forceinline__ void substitute(const float* src, uint16_t* dst, int k0, int app_pos, int app_len,
                                             int wlo, int whi, int d, int tid, int ring_start, int S,
                                             int col0 = 0) {
    // An opaque copy of the thread index: the chunk arithmetic below then
    // cannot be hoisted out of this rarely taken branch into the key loop,
    // where it would hold registers.
    int t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(tid));
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = t + it * NT;
      const int j = k0 + c / CH, col = col0 + (c % CH) * 8;
      const int i = j - app_pos;
      if ((TOTAL % NT == 0 || c < TOTAL) && col < d && (unsigned)i < (unsigned)app_len) {
        const float* f = src + (size_t)i * d + col;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(f);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(f + 4);
        const u32x4 v = {Elem<T>::pack2(lo[0], lo[1]), Elem<T>::pack2(lo[2], lo[3]),
                         Elem<T>::pack2(hi[0], hi[1]), Elem<T>::pack2(hi[2], hi[3])};
        r[it] = v;
        if (dst && i >= wlo && i < whi) {
          int slot = j;
          if (ring_start >= 0) {
            slot = ring_start + j;
            slot -= (slot >= S) ? S : 0;
          }
          *reinterpret_cast<u32x4*>(dst + (size_t)slot * d + col) = v;
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* sm, int tid) const {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = tid + it * NT;
      if (TOTAL % NT == 0 || c < TOTAL)
        *reinterpret_cast<u32x4*>(sm + (c / CH) * PITCH + (c % CH) * 8) = r[it];
    }
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// x / d for 0 <= x < 2^31 with the launch's precomputed (m, s) for d: one
// multiply-high and a shift instead of a divide sequence (see FastDiv).
__device__ __forceinline__ int fdiv(int x, FastDiv f) {
  return (int)(((uint64_t)(uint32_t)x * f.m) >> (31 + f.s));
}
// Raw buffer descriptor words (base, stride 0, num_records = bytes, the same
// format word as make_rsrc) for the inline-assembly load below.
__device__ __forceinline__ u32x4 raw_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// The same 16-byte direct-to-LDS buffer load, written as inline assembly so
// that the compiler does not track it: the compiler treats a direct-to-LDS
// load as a store to any LDS location and makes every later LDS read wait
// for it.  Here the caller orders the loads and the reads itself, with an
// explicit vmcnt wait and a workgroup barrier before the stage is read.  The
// instruction has no register result; its operands are read at issue.
__device__ __forceinline__ void lds_dma16_async(const u32x4& rs, uint16_t* lds, int voff) {
  const uint32_t m0 = wave_uniform(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  // (s_nop: one wait state between the write of M0 and the load that reads it.)
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rs), "{m0}"(m0) : "memory");
}


// Transposed 4-key x 1-column read (see above); returns the 4 keys of this
// lane's column as two packed dwords.
__device__ __forceinline__ u32x2 lds_read_tr4(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

constexpr int kKPad = 16;  // elements of padding after each staged K row

// Per-wave tile work of the register-staged kernels (prefill_kernel,
// splitkv_kernel).  A step is 32 keys: S^T blocks hh = 0, 1 of 16 keys each,
// natural key order (block row rho is key kbase + 16*hh + rho), so lane group
// g4 holds keys 4*g4 + i (hh = 0) and 16 + 4*g4 + i (hh = 1): the P^T operand
// that the transposed V reads above produce.  K and V rows are padded to KP /
// VP elements in LDS, which puts the rows of one fragment read on distinct
// banks.  K rows take 32 bytes of padding (kKPad): with 16, the K fragment
// reads of the split-KV kernel still conflicted (SQ_LDS_BANK_CONFLICT
// 524288 per launch of the 4:1 decode, 0 with 32; 44.1 -> 43.8 us).

// One 32-key step: scores, softcap, mask, online softmax and P.V; each
// fragment is read from LDS right before its products.  The MASK instance
// applies the mask only when rmask is set (a run-time choice between full and
// partial tiles within one copy of the code).
template <typename T, int DQK, int DV, int NQB, int KP, int VP, bool SOFTCAP, bool MASK>
__device__ __forceinline__ void tile_step(const uint16_t* Ks, const uint16_t* Vs, int kbase, int kglob0,
                                          const u32x4 (&qf)[NQB][DQK], const int (&qpos)[NQB],
                                          float (&m_e)[NQB], f32x4 (&ls)[NQB], f32x4 (&o)[NQB][DV],
                                          const KernelArgs& a, int c16, int g4, bool rmask = true) {
  // ---- S^T = K Q^T -------------------------------------------------------
  f32x4 s[NQB][2];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) s[qb][0] = s[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint16_t* krow = Ks + (kbase + 16 * hh + c16) * KP;
#pragma unroll
    for (int t = 0; t < DQK; ++t) {
      const u32x4 k1 = *reinterpret_cast<const u32x4*>(krow + 8 * g4 + 32 * t);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s[qb][hh] = Elem<T>::mfma(k1, qf[qb][t], s[qb][hh]);
    }
  }

  // ---- softcap, mask, online softmax, P^T ------------------------------------
  // Row maxima of every row block first; the accumulators are rescaled under
  // one wave-uniform branch (rows whose maximum did not grow by more than the
  // slack are multiplied by exactly 1), so the products and exponentials of
  // all row blocks form one straight-line block.
  float mxe[NQB];
  bool grow = false;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    if (MASK && rmask) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kglob0 + kbase + 16 * hh + 4 * g4 + i;
          if (!key_visible(j, qpos[qb], a.Lkv, a.causal, a.window)) s[qb][hh][i] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][hh][i]);
    mx = col_max(mx);
    if (SOFTCAP) {
      // Same formula as the per-score path below, so the row maximum maps to
      // exactly 2^0 before any rescale slack.
      mxe[qb] = (mx == kNegInf) ? kNegInf
                                : __builtin_fmaf(fast_rcp(fast_exp2(mx * a.gamma) + 1.0f), -2.0f * a.c2, a.c2);
    } else {
      mxe[qb] = mx * a.alpha;
    }
    grow = grow || (mxe[qb] > m_e[qb] + kRescaleSlack);
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const bool up = mxe[qb] > m_e[qb] + kRescaleSlack;
      const float f = up ? fast_exp2(m_e[qb] - mxe[qb]) : 1.0f;  // 0 when m_e was -inf
      if (up) m_e[qb] = mxe[qb];
      ls[qb] *= f;
#pragma unroll
      for (int db = 0; db < DV; ++db) o[qb][db] *= f;
    }
  }
  u32x4 pk[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float mref = (m_e[qb] == kNegInf) ? 0.f : m_e[qb];
    float p[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = s[qb][hh][i];
        float pv;
        if (SOFTCAP) {
          // c*tanh(u) = c - 2c/(exp(2u)+1); in base-2 units the exponent is
          // c2 - 2*c2*r - mref with r = 1/(2^(x*gamma) + 1).
          const float r = fast_rcp(fast_exp2(x * a.gamma) + 1.0f);
          pv = fast_exp2(__builtin_fmaf(r, -2.0f * a.c2, a.c2 - mref));
          if (MASK && x == kNegInf) pv = 0.f;
        } else {
          pv = fast_exp2(__builtin_fmaf(x, a.alpha, -mref));
        }
        p[hh * 4 + i] = pv;
      }
    pk[qb] = u32x4{Elem<T>::pack2(p[0], p[1]), Elem<T>::pack2(p[2], p[3]),
                   Elem<T>::pack2(p[4], p[5]), Elem<T>::pack2(p[6], p[7])};
  }
  // Row sums on the matrix cores from the same 16-bit probabilities that
  // enter P.V (an all-ones A operand): every lane of column c16 receives the
  // sum over the step's 32 keys, so a constant V comes back exactly.
  {
    const u32x4 ones = {OnesOperand<T>::kPair, OnesOperand<T>::kPair, OnesOperand<T>::kPair,
                        OnesOperand<T>::kPair};
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) ls[qb] = Elem<T>::mfma(ones, pk[qb], ls[qb]);
  }

  // ---- O^T += V^T P^T ---------------------------------------------------------
  const uint16_t* v0 = Vs + (kbase + 4 * g4 + (c16 >> 2)) * VP + 4 * (c16 & 3);
  const uint16_t* v1 = v0 + 16 * VP;
#pragma unroll
  for (int db = 0; db < DV; ++db) {
    const u32x2 lo = lds_read_tr4(v0 + 16 * db);
    const u32x2 hi = lds_read_tr4(v1 + 16 * db);
    const u32x4 vf1 = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) o[qb][db] = Elem<T>::mfma(vf1, pk[qb], o[qb][db]);
  }
}

// Both 32-key steps of a 64-key tile.
template <typename T, int DQK, int DV, int NQB, int KP, int VP, bool SOFTCAP>
__device__ __forceinline__ void tile_pair(const uint16_t* Ks, const uint16_t* Vs, int k0, bool full,
                                          const u32x4 (&qf)[NQB][DQK], const int (&qpos)[NQB],
                                          float (&m_e)[NQB], f32x4 (&ls)[NQB], f32x4 (&o)[NQB][DV],
                                          const KernelArgs& a, int c16, int g4) {
#pragma unroll
  for (int kb = 0; kb < 64; kb += 32) {
    if (full)
      tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, false>(Ks, Vs, kb, k0, qf, qpos, m_e, ls, o, a, c16, g4);
    else
      tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, true>(Ks, Vs, kb, k0, qf, qpos, m_e, ls, o, a, c16, g4);
  }
}

// ---------------------------------------------------------------------------
// Prefill / encoder kernel: one workgroup per (batch, kv head, block of m
// query positions); NWAVES waves x NQB x 16 rows; rows are (head of the group,
// position) pairs with the head index fastest.  Two LDS stages: while every
// wave works on one tile, the next tile's loads are in flight in registers and
// are written to the other stage right after, so one barrier per tile.
// ---------------------------------------------------------------------------
template <typename T, int DQK, int DV, int NQB, int NWAVES, bool SOFTCAP>
__global__ __launch_bounds__(NWAVES * 64) void prefill_kernel(KernelArgs a) {
  constexpr int NT = NWAVES * 64;
  constexpr int KEYS = kPrefillKeys;
  constexpr int KP = DQK * 32 + kKPad;  // 16 rows of a K read land on distinct banks
  constexpr int VP = DV * 16 + 16;      // 4 rows x 32 B of a transposed V read do too
  constexpr int STAGE = KEYS * (KP + VP);
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  Timeline tl(NWAVES);
  tl.mark<0>();

  // Every argument the first loads depend on, asked for at once, so that
  // their loads leave in one batch and cost one round trip.
  asm volatile("" : : "s"(a.kv_stride), "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.n_pos_blk), "s"(a.Hkv), "s"(a.Hq),
               "s"(a.G), "s"(a.m), "s"(a.Lq), "s"(a.Lkv), "s"(a.causal), "s"(a.window), "s"(a.div_g.m),
               "s"(a.div_g.s), "s"(a.div_npos.m), "s"(a.div_npos.s), "s"(a.div_hkv.m), "s"(a.div_hkv.s),
               "s"(a.nwg));
  const int bid = blockIdx.x;
  const int unit = fdiv(bid, a.div_npos);  // b * Hkv + kvh
  const int pblk = a.n_pos_blk - 1 - (bid - unit * a.n_pos_blk);  // longest key bands first (causal)
  const int b = fdiv(unit, a.div_hkv), kvh = unit - b * a.Hkv;
  const int G = a.G, d = a.d;
  const int q0 = pblk * a.m;
  const int m_eff = min(a.m, a.Lq - q0);
  const int off = a.Lkv - a.Lq;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (size_t)unit * a.kv_stride;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (size_t)unit * a.kv_stride;
  uint16_t* og = static_cast<uint16_t*>(a.out);

  u32x4 qf[NQB][DQK];
  int qpos[NQB];
  bool rok[NQB];
  size_t roff[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = (wave * NQB + qb) * 16 + c16;
    const int pl = fdiv(r, a.div_g), hr = r - pl * G;
    rok[qb] = pl < m_eff;
    const int pos = q0 + pl;
    qpos[qb] = pos + off;
    const int head = kvh * G + hr;
    roff[qb] = (((size_t)b * a.Hq + head) * a.Lq + (rok[qb] ? pos : 0)) * d;
    load_q<DQK>(qf[qb], qg + roff[qb], rok[qb], d, g4);
  }

  // Key band of this block of positions.
  const int pos_min = q0 + off, pos_max = q0 + m_eff - 1 + off;
  int key_lo = 0, key_hi = a.Lkv - 1;
  if (a.causal) key_hi = min(key_hi, pos_max);
  if (a.window > 0) {
    key_lo = max(0, pos_min - a.window + 1);
    if (!a.causal) key_hi = min(key_hi, pos_max + a.window - 1);
  }
  const int t_begin = key_lo / KEYS, t_end = key_hi / KEYS + 1;

  float m_e[NQB];
  f32x4 ls[NQB], o[NQB][DV];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_e[qb] = kNegInf;
    ls[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DV; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  RowTile<KEYS, DQK * 4, KP, NT> kt;
  RowTile<KEYS, DV * 2, VP, NT> vt;
  kt.init(d, tid);
  vt.init(d, tid);
  kt.load(kg, t_begin * KEYS, a.Lkv, d);
  vt.load(vg, t_begin * KEYS, a.Lkv, d);
  kt.store(smem, tid);
  vt.store(smem + KEYS * KP, tid);
  __syncthreads();
  tl.mark<1>();
  for (int t = t_begin; t < t_end; ++t) {
    const int k0 = t * KEYS;
    const int cur = (t - t_begin) & 1;
    const uint16_t* Ks = smem + cur * STAGE;
    const uint16_t* Vs = Ks + KEYS * KP;
    if (t + 1 < t_end) {
      kt.load(kg, k0 + KEYS, a.Lkv, d);
      vt.load(vg, k0 + KEYS, a.Lkv, d);
    }
    bool full = k0 + KEYS <= a.Lkv;
    if (a.causal) full = full && (k0 + KEYS - 1 <= pos_min);
    if (a.window > 0) {
      full = full && (pos_max - k0 < a.window);
      if (!a.causal) full = full && (k0 + KEYS - 1 - pos_min < a.window);
    }
    // Two 32-key steps per tile; K fragments of the second step are read
    // during the first step's products.
    tile_pair<T, DQK, DV, NQB, KP, VP, SOFTCAP>(Ks, Vs, k0, full, qf, qpos, m_e, ls, o, a, c16, g4);
    if (t + 1 < t_end) {
      uint16_t* nxt = smem + (cur ^ 1) * STAGE;
      kt.store(nxt, tid);
      vt.store(nxt + KEYS * KP, tid);
    }
    __syncthreads();
  }
  tl.mark<2>();

#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
    if (rok[qb]) store_row<T, DV>(og + roff[qb], o[qb], 1.0f / ls[qb][0], d, g4);
  tl.mark<7>();
  tl.flush();
}

// ---------------------------------------------------------------------------
// Software-pipelined prefill for head size 128.
//
// The key axis is walked in 32-key steps j.  Step j runs, in straight-line
// code,
//   * the fp32 softmax arithmetic of the scores S_j (vector ALU),
//   * the MFMA products of the next step's scores S_{j+1} = K_{j+1} Q^T,
//   * the MFMA products of the previous step's O^T += V_{j-1}^T P_{j-1}^T,
// so the matrix cores work while the vector ALU computes probabilities.  The
// row sum of P is taken on the matrix cores too (an all-ones A operand), from
// the same 16-bit probabilities that enter P.V.
//
// Fixed reference (FIXREF): with a softcap c, every score lies in [-c, c], so
// exp2 of a softcapped score (base-2 units) minus c*log2(e) - 64 lies in
// [2^(64 - 2c log2 e), 2^64].  For c <= 57.5 (c*log2(e) <= 83) the smallest
// probability is at least 2^-102: its products with values down to 2^-24
// inside P.V stay in the normal range of fp32, and the largest, 2^64, leaves
// room for sums over 2^23 keys and values up to 2^40.  No running maximum and
// no rescale are needed.  Otherwise the running maximum is kept with the lazy
// rescale.
//
// Workgroup: four waves (one per SIMD), 128 rows, one 32-key tile per step.
// LDS holds five stages of one K and one V tile (16 KB per stage pair), all
// K tiles first, then all V tiles, filled by direct global-to-LDS loads: two
// workgroups fit in one CU, so every SIMD runs waves of two independent
// workgroups whose barriers and load waits do not line up.  Tile j+3 is
// requested once every wave is past step j-1 (the last reader of tile j-2's
// stage), two steps before it is first read.  The step loop is unrolled over
// the five stages, so every fragment read is one of twelve per-lane base
// addresses plus a constant offset.
// ---------------------------------------------------------------------------
constexpr int kPipe4Stages = 5;
constexpr int kPipe4Tile = 32 * 128;                       // elements of one K or V tile
constexpr int kPipe4VRegion = kPipe4Stages * kPipe4Tile;  // first V tile (elements)


// Per-lane fragment offsets (elements): ka[t] -> K row c16, chunk 4t+g4 of
// tile row 0 (swizzled slot); va[db] -> the transposed V read of columns
// 16*db.. of tile row 4*g4 + c16/4.
struct PipeAddr {
  int ka[4];
  int va[8];
};

// Probabilities of scores I0 .. I0+N-1 of 4 (one 16-key half of one 16-row
// block), fp32.
template <bool SOFTCAP, int I0 = 0, int N = 4>
__device__ __forceinline__ void pipe_probs(const f32x4& x, float mref, const KernelArgs& a, float (&p)[4]) {
  if (SOFTCAP) {
    // Stage by stage over the N scores, so that N independent chains of
    // dependent transcendentals are in flight instead of one.
    float t[4];
#pragma unroll
    for (int i = I0; i < I0 + N; ++i) t[i] = fast_exp2(x[i] * a.gamma);
#pragma unroll
    for (int i = I0; i < I0 + N; ++i) t[i] = fast_rcp(t[i] + 1.0f);
#pragma unroll
    for (int i = I0; i < I0 + N; ++i) p[i] = fast_exp2(__builtin_fmaf(t[i], -2.0f * a.c2, a.c2 - mref));
  } else {
#pragma unroll
    for (int i = I0; i < I0 + N; ++i) p[i] = fast_exp2(__builtin_fmaf(x[i], a.alpha, -mref));
  }
}

// Keeps the compiler from moving the computation of v across this point
// (it sees v as read and rewritten here).
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(f32x4& v) { asm volatile("" : "+v"(v)); }

// One 32-key step.  Kst + KOFF: step j+1's K rows (stage array, tile row),
// Vst + VOFF: step j-1's V rows.  sc: scores of step j (in), sn: of
// step j+1 (out); pp: probabilities of step j-1 (in), pc: of step j (out).
// Visibility of key kglob + 16*hh + 4*g4 + i to row block qb:
// (unsigned)(ubase[qb] + 16*hh + i) <= span[qb]; MASK is false when every
// key of the step is visible to every row of the workgroup.
//
// NQB 16-row blocks per wave (2, or 1 for half-height blocks).  The products
// and the exponentials form one straight-line block of four quarters, each
// with 4*NQB MFMAs (two V and two K fragments) and the probabilities of 2*NQB
// scores, so that few fragments are live at a time.  The
// mask (partial steps only) is applied after that block.  With a running
// maximum, the new maximum is taken first (the exponentials use it at once)
// and the accumulators are rescaled at the end, after the products of step
// j-1 -- whose probabilities used the old maximum -- are in.
template <typename T, int NQB, bool SOFTCAP, bool FIXREF, int KOFF, int VOFF>
__device__ __forceinline__ void pipe_step(bool mask, const uint16_t* Kst, const uint16_t* Vst, const PipeAddr& ad,
                                          f32x4 (&sc)[NQB][2], f32x4 (&sn)[NQB][2],
                                          const u32x4 (&pp)[NQB], u32x4 (&pc)[NQB], const u32x4 (&qf)[NQB][4],
                                          f32x4 (&o)[NQB][8], f32x4 (&ls)[NQB], float (&m_e)[NQB],
                                          const int (&ubase)[NQB], const int (&span)[NQB], const KernelArgs& a) {
  const u32x4 ones = {OnesOperand<T>::kPair, OnesOperand<T>::kPair, OnesOperand<T>::kPair,
                      OnesOperand<T>::kPair};
  float mref[NQB], resc[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) resc[qb] = 1.0f;
  if constexpr (FIXREF) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mref[qb] = a.c2 - 64.0f;
  } else {
    if (mask) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((unsigned)(ubase[qb] + 16 * hh + i) > (unsigned)span[qb]) sc[qb][hh][i] = kNegInf;
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = fmaxf(fmaxf(fmaxf(sc[qb][0][0], sc[qb][0][1]), fmaxf(sc[qb][0][2], sc[qb][0][3])),
                       fmaxf(fmaxf(sc[qb][1][0], sc[qb][1][1]), fmaxf(sc[qb][1][2], sc[qb][1][3])));
      mx = col_max(mx);
      float mxe;
      if (SOFTCAP)
        mxe = (mx == kNegInf) ? kNegInf
                              : __builtin_fmaf(fast_rcp(fast_exp2(mx * a.gamma) + 1.0f), -2.0f * a.c2, a.c2);
      else
        mxe = mx * a.alpha;
      if (mxe > m_e[qb] + kRescaleSlack) {
        resc[qb] = fast_exp2(m_e[qb] - mxe);  // 0 when m_e was -inf
        m_e[qb] = mxe;
      }
      mref[qb] = (m_e[qb] == kNegInf) ? 0.f : m_e[qb];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // Fragments of quarter k: V columns 32k..32k+31 of step j-1 and K chunks
  // 2(k%2), 2(k%2)+1 of key rows 16(k/2).. of step j+1.  Each quarter reads
  // the next quarter's fragments before its own products.
  auto frags = [&](int k, u32x4 (&vf)[2], u32x4 (&kf)[2]) {
    const int hh = k >> 1, t0 = 2 * (k & 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint16_t* v0 = Vst + ad.va[2 * k + e] + VOFF;
      const u32x2 lo = lds_read_tr4(v0);
      const u32x2 hi = lds_read_tr4(v0 + 16 * 128);
      vf[e] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      kf[e] = *reinterpret_cast<const u32x4*>(Kst + ad.ka[t0 + e] + KOFF + hh * 16 * 128);
    }
  };
  float p[NQB][2][4];
  u32x4 fr[2][2][2];  // [buffer][V, K][e]
  frags(0, fr[0][0], fr[0][1]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int hh = k >> 1, t0 = 2 * (k & 1);
    // Scores whose probabilities this quarter computes: of block qs, half hs
    // (two row blocks: all four of a half per quarter; one row block: two).
    constexpr bool TWO = NQB == 2;
    const int qs = TWO ? (k >> 1) : 0, hs = TWO ? (k & 1) : (k >> 1);
    const int cur = k & 1;
    pin(sc[qs][hs]);
    if (k < 3) frags(k + 1, fr[cur ^ 1][0], fr[cur ^ 1][1]);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) o[qb][2 * k + e] = Elem<T>::mfma(fr[cur][0][e], pp[qb], o[qb][2 * k + e]);
    if (k == 3) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) ls[qb] = Elem<T>::mfma(ones, pp[qb], ls[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x4 acc = (k & 1) ? sn[qb][hh] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 2; ++e) acc = Elem<T>::mfma(fr[cur][1][e], qf[qb][t0 + e], acc);
      sn[qb][hh] = acc;
    }
    if constexpr (TWO) {
      pipe_probs<SOFTCAP>(sc[qs][hs], mref[qs], a, p[qs][hs]);
#pragma unroll
      for (int i = 0; i < 4; ++i) pin(p[qs][hs][i]);
    } else if (k & 1) {
      pipe_probs<SOFTCAP, 2, 2>(sc[qs][hs], mref[qs], a, p[qs][hs]);
      pin(p[qs][hs][2]);
      pin(p[qs][hs][3]);
    } else {
      pipe_probs<SOFTCAP, 0, 2>(sc[qs][hs], mref[qs], a, p[qs][hs]);
      pin(p[qs][hs][0]);
      pin(p[qs][hs][1]);
    }
    // Next quarter's fragment reads first, then one MFMA per three vector-ALU ops.
    if (k < 3) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int g = 0; g < 5 * NQB; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  if (mask) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((unsigned)(ubase[qb] + 16 * hh + i) > (unsigned)span[qb]) p[qb][hh][i] = 0.f;
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
    pc[qb] = u32x4{Elem<T>::pack2(p[qb][0][0], p[qb][0][1]), Elem<T>::pack2(p[qb][0][2], p[qb][0][3]),
                   Elem<T>::pack2(p[qb][1][0], p[qb][1][1]), Elem<T>::pack2(p[qb][1][2], p[qb][1][3])};

  if constexpr (!FIXREF) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
      if (resc[qb] != 1.0f) {
        ls[qb] *= resc[qb];
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qb][db] *= resc[qb];
      }
  }
}

// ---------------------------------------------------------------------------
// The pipelined prefill kernel for head size 128 (layout and schedule above).
//
// pipe4_block: one block of 64*NQB rows -- query positions q0 .. q0+m_item-1
// of unit `unit` (batch row * Hkv + kv head), every head of the group, head
// fastest -- through its whole key band.  A workgroup that runs two blocks
// places a barrier between them: the second block's first loads overwrite
// stages the first block's last steps read.
// ---------------------------------------------------------------------------
template <typename T, int NQB, bool SOFTCAP, bool FIXREF>
__device__ __forceinline__ void pipe4_block(const KernelArgs& a, uint16_t* smem, int unit, int q0, int m_item,
                                            Timeline& tl, bool second) {
  constexpr int NWAVES = 4, D = 128, KEYS = 32, TILE = kPipe4Tile, NS = kPipe4Stages;
  constexpr int IPW = KEYS / 4 / NWAVES;  // 4-row direct-to-LDS loads per wave per tensor
  static_assert(IPW == 2, "the wait counts below assume two loads per tensor per wave");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int g4 = lane >> 4, c16 = lane & 15;
  const int b = fdiv(unit, a.div_hkv), kvh = unit - b * a.Hkv;
  const int G = a.G;
  const int m_eff = min(m_item, a.Lq - q0);
  const int off = a.Lkv - a.Lq;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (size_t)unit * a.kv_stride;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (size_t)unit * a.kv_stride;
  uint16_t* og = static_cast<uint16_t*>(a.out);

  // Key band of this block of positions, in tiles.
  const int pos_min = q0 + off, pos_max = q0 + m_eff - 1 + off;
  int key_lo = 0, key_hi = a.Lkv - 1;
  if (a.causal) key_hi = min(key_hi, pos_max);
  if (a.window > 0) {
    key_lo = max(0, pos_min - a.window + 1);
    if (!a.causal) key_hi = min(key_hi, pos_max + a.window - 1);
  }
  const int t_begin = key_lo / KEYS, t_end = key_hi / KEYS + 1;

  // Q first: the direct-to-LDS loads are counted after it, so waiting for
  // the first tile also waits for Q.
  u32x4 qf[NQB][4];
  int rconst[NQB], span[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = (wave * NQB + qb) * 16 + c16;
    const int pl = fdiv(r, a.div_g), hr = r - pl * G;
    const bool ok = pl < m_eff;
    const int pos = q0 + pl + off;
    const size_t ro = (((size_t)b * a.Hq + kvh * G + hr) * a.Lq + (ok ? q0 + pl : 0)) * D;
    load_q<4>(qf[qb], qg + ro, ok, D, g4);
    // Visible keys of this row: [lo, hi].
    const int lo = a.window > 0 ? pos - a.window + 1 : 0;
    int hi = a.Lkv - 1;
    if (a.causal) hi = min(hi, pos);
    else if (a.window > 0) hi = min(hi, pos + a.window - 1);
    rconst[qb] = 4 * g4 - lo;
    span[qb] = hi - lo;
  }

  int voffK[IPW], voffV[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int row = 4 * (wave * IPW + j) + (lane >> 4), slot = lane & 15;
    voffK[j] = (row * D + ((slot ^ (row & 15)) << 3)) * 2;
    voffV[j] = (row * D + ((slot ^ (2 * (row & 7))) << 3)) * 2;
  }
  uint16_t* const sk = smem;
  uint16_t* const sv = smem + kPipe4VRegion;
  auto fetch = [&](int t, int st) {
    // (Forced into scalar registers: the descriptor must be uniform.)
    const int k0 = wave_uniform(t * KEYS);
    const uint32_t bytes = (uint32_t)wave_uniform((int)((uint32_t)(a.Lkv - k0) * (uint32_t)(D * 2)));
    const u32x4 rk = raw_rsrc(kg + (size_t)k0 * D, bytes);
    const u32x4 rv = raw_rsrc(vg + (size_t)k0 * D, bytes);
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int row0 = st * TILE + (wave * IPW + j) * 4 * D;
      lds_dma16_async(rk, sk + row0, voffK[j]);
      lds_dma16_async(rv, sv + row0, voffV[j]);
    }
  };

  // Tiles t_begin .. t_begin+2 into stages 0..2.
  fetch(t_begin, 0);
  if (t_begin + 1 < t_end) fetch(t_begin + 1, 1);
  if (t_begin + 2 < t_end) fetch(t_begin + 2, 2);
  // The last stage's V tile stands in for "the tile before the first" (with
  // zero probabilities): clear it so that it holds finite values.
  {
    uint16_t* z = sv + (NS - 1) * TILE;
#pragma unroll
    for (int i = 0; i < TILE / (8 * 256); ++i)
      *reinterpret_cast<u32x4*>(z + (i * 256 + tid) * 8) = u32x4{0u, 0u, 0u, 0u};
  }

  PipeAddr ad;
#pragma unroll
  for (int t = 0; t < 4; ++t) ad.ka[t] = c16 * 128 + (((4 * t + g4) ^ c16) << 3);
  {
    const int row = 4 * g4 + (c16 >> 2);
    const int sw = 2 * (row & 7);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      ad.va[db] = row * 128 + (((2 * db + ((c16 & 3) >> 1)) ^ sw) << 3) + 4 * (c16 & 1);
  }

  // Tiles t_begin and t_begin+1 in LDS (t_begin+2 may still fly).
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (t_begin + 2 < t_end)
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (second) tl.mark<4>();
  else tl.mark<1>();

  float m_e[NQB];
  f32x4 o[NQB][8], ls[NQB];
  f32x4 sa[NQB][2], sb[NQB][2];
  u32x4 pa[NQB], pb[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_e[qb] = kNegInf;
    ls[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    pb[qb] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int db = 0; db < 8; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Scores of the first step (stage 0).
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc = Elem<T>::mfma(*reinterpret_cast<const u32x4*>(sk + ad.ka[t] + hh * 16 * 128), qf[qb][t], acc);
      sa[qb][hh] = acc;
    }

  // Integer flags and an explicit wave-uniform result keep the test in
  // scalar registers (as booleans it was built as a lane mask in vector
  // registers on every step).
  auto step_full = [&](int kg0) {
    int full = kg0 + KEYS <= a.Lkv;
    full &= (a.causal == 0) | (kg0 + KEYS - 1 <= pos_min);
    full &= (a.window <= 0) | ((pos_max - kg0 < a.window) & ((a.causal != 0) | (kg0 + KEYS - 1 - pos_min < a.window)));
    return __builtin_amdgcn_readfirstlane(full) != 0;
  };
  // Step t (tile t in stage ST, compile time): softmax of tile t, scores of
  // tile t+1 (stage ST+1; discarded after the last tile), P.V of tile t-1
  // (stage ST-1).  Before it: tile t+1 landed, and every wave past step t-1.
  // sc/sn/pp/pc alternate between the two register sets from step to step.
  auto step = [&](auto stc, int t, f32x4 (&sc)[NQB][2], f32x4 (&sn)[NQB][2], const u32x4 (&pp)[NQB],
                  u32x4 (&pc)[NQB]) {
    constexpr int ST = decltype(stc)::value;
    constexpr int SP = (ST + NS - 1) % NS, SN = (ST + 1) % NS;
    if (t > t_begin) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (t + 2 < t_end)
        __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): tile t+2 may still fly
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __syncthreads();
    }
    // Tile t-2's stage is free: every wave is past step t-1, its last reader.
    if (t + 3 < t_end) fetch(t + 3, (ST + 3) % NS);
    const int kg0 = t * KEYS;
    int ub[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) ub[qb] = kg0 + rconst[qb];
    pipe_step<T, NQB, SOFTCAP, FIXREF, SN * TILE, SP * TILE>(!step_full(kg0), sk, sv, ad, sc, sn, pp, pc, qf, o,
                                                             ls, m_e, ub, span, a);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  using S4 = std::integral_constant<int, 4>;
  // Ten steps per turn: five stages, two register sets.
  int t = t_begin, last = 0;
  while (true) {
    step(S0{}, t, sa, sb, pb, pa);
    if (++t >= t_end) { last = 0; break; }
    step(S1{}, t, sb, sa, pa, pb);
    if (++t >= t_end) { last = 1; break; }
    step(S2{}, t, sa, sb, pb, pa);
    if (++t >= t_end) { last = 2; break; }
    step(S3{}, t, sb, sa, pa, pb);
    if (++t >= t_end) { last = 3; break; }
    step(S4{}, t, sa, sb, pb, pa);
    if (++t >= t_end) { last = 4; break; }
    step(S0{}, t, sb, sa, pa, pb);
    if (++t >= t_end) { last = 5; break; }
    step(S1{}, t, sa, sb, pb, pa);
    if (++t >= t_end) { last = 6; break; }
    step(S2{}, t, sb, sa, pa, pb);
    if (++t >= t_end) { last = 7; break; }
    step(S3{}, t, sa, sb, pb, pa);
    if (++t >= t_end) { last = 8; break; }
    step(S4{}, t, sb, sa, pa, pb);
    if (++t >= t_end) { last = 9; break; }
  }
  if (second) tl.mark<5>();
  else tl.mark<2>();
  // P.V and row sums of the last tile (its probabilities are in pa after an
  // even-numbered step of the turn, in pb after an odd one).
  {
    const u32x4 ones = {OnesOperand<T>::kPair, OnesOperand<T>::kPair, OnesOperand<T>::kPair,
                        OnesOperand<T>::kPair};
    u32x4 pfin[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) pfin[qb] = (last & 1) ? pb[qb] : pa[qb];
    const int vst = (last % NS) * TILE;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* v0 = sv + ad.va[db] + vst;
      const u32x2 lo = lds_read_tr4(v0);
      const u32x2 hi = lds_read_tr4(v0 + 16 * 128);
      const u32x4 v1 = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) o[qb][db] = Elem<T>::mfma(v1, pfin[qb], o[qb][db]);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) ls[qb] = Elem<T>::mfma(ones, pfin[qb], ls[qb]);
  }

#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = (wave * NQB + qb) * 16 + c16;
    const int pl = fdiv(r, a.div_g), hr = r - pl * G;
    if (pl < m_eff) {
      const size_t ro = (((size_t)b * a.Hq + kvh * G + hr) * a.Lq + q0 + pl) * D;
      store_row<T, 8>(og + ro, o[qb], 1.0f / ls[qb][0], D, g4);
    }
  }
  if (second) tl.mark<6>();
  else tl.mark<3>();
}

// Work items of one unit, in launch order (item j; n = n_pos_blk blocks of m
// positions, R = pf_ramp):
//   j <  pf_pairs:             blocks R-1-j and j, one after the other (one
//                              block when the two coincide);
//   j <  pf_pairs + pf_full:   block n-1-(j-pf_pairs) (whole blocks, last first);
//   otherwise:                 the halves (m/2 positions, one 16-row block per
//                              wave) of the remaining blocks, two items each.
// Under a causal mask the first R blocks have shorter key bands than the
// rest (the ramp); pairing its two ends gives items of about one full band.
// The host sets the counts from a model of the launch so that the last
// round of workgroups holds the half-size items.
template <typename T, bool SOFTCAP, bool FIXREF>
__global__ __launch_bounds__(256, 2) void prefill_pipe4_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kPipe4Stages * kPipe4Tile];
  Timeline tl(kPipe4Waves);
  tl.mark<0>();
  // Every argument the first loads depend on, asked for at once, so that
  // their loads leave in one batch and cost one round trip.
  asm volatile("" : : "s"(a.kv_stride), "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.n_pos_blk), "s"(a.Hkv), "s"(a.Hq),
               "s"(a.G), "s"(a.m), "s"(a.Lq), "s"(a.Lkv), "s"(a.causal), "s"(a.window), "s"(a.div_g.m),
               "s"(a.div_g.s), "s"(a.div_items.m), "s"(a.div_items.s), "s"(a.div_hkv.m), "s"(a.div_hkv.s),
               "s"(a.nwg), "s"(a.pf_items), "s"(a.pf_pairs), "s"(a.pf_ramp), "s"(a.pf_full));
  // Workgroups are dealt to the 8 XCDs round robin (workgroup i to XCD i % 8),
  // each XCD with its own L2.  Renumber so that every XCD gets a contiguous
  // range of (unit, item) pairs: the items of one unit then share their K/V
  // tiles in one L2.
  const int bid = blockIdx.x;
  int lin = bid;
  if ((a.nwg & 7) == 0) lin = (bid & 7) * (a.nwg >> 3) + (bid >> 3);
  const int unit = fdiv(lin, a.div_items);
  const int j = lin - unit * a.pf_items;
  const int whole = a.pf_pairs + a.pf_full;
  if (j >= whole) {
    const int h = j - whole, half = a.m >> 1;
    const int pblk = a.n_pos_blk - 1 - a.pf_full - (h >> 1);
    pipe4_block<T, 1, SOFTCAP, FIXREF>(a, smem, unit, pblk * a.m + (h & 1) * half, half, tl, false);
    tl.mark<7>();
    tl.flush();
    return;
  }
  int pb0 = a.n_pos_blk - 1 - (j - a.pf_pairs), pb1 = -1;
  if (j < a.pf_pairs) {
    pb0 = a.pf_ramp - 1 - j;
    if (j < pb0) pb1 = j;
  }
  // At most two passes; one copy of the block code.
  bool second = false;
  while (true) {
    pipe4_block<T, 2, SOFTCAP, FIXREF>(a, smem, unit, pb0 * a.m, a.m, tl, second);
    if (pb1 < 0) break;
    pb0 = pb1;
    pb1 = -1;
    second = true;
    __syncthreads();
  }
  tl.mark<7>();
  tl.flush();
}

// ---------------------------------------------------------------------------
// Split-KV kernel (decode, multi-token decode, short and mid-length
// sequences): one workgroup of NW waves per (unit = batch*Hkv + kv head, block
// of m query positions, key split).  Its rows are (position, head of the group)
// pairs, head fastest: NQB blocks of 16, m*G <= 16*NQB of them real.  Each
// 32*NW-key tile is staged once (K and V row-major, V read transposed); wave w
// takes keys [32w, 32w+32) of it for all rows, so the key axis is split across
// the waves.  The wave states are merged in LDS in wave order.  With one
// split the merged rows are the output; otherwise the split's partial is
// written and the last split to arrive for the block merges all partials in
// split order.  NW is 4 (128-key tiles), or 8 (256-key tiles, two waves per
// SIMD) for a single 16-row block with long key ranges per workgroup and for
// three 16-row blocks over an unsplit band of four or more 128-key tiles.  With
// many splits of one 16-row block the key range of a split is shared by two
// workgroups (NCOL = 2), each with half of V's columns (DV is then the half's
// width); each half merges its own partials.  A decode step with the KV-cache
// update folded in (TensorTonic, "KV Cache Update at a Position") passes the
// new rows as float32 inputs: the tiles holding them take them from there,
// and one workgroup per new key writes it to its cache slot.
// ---------------------------------------------------------------------------
template <typename T, int DQK, int DV, int NQB, int NW, bool SOFTCAP, bool RING, int NCOL, bool STREAM>
__global__ __launch_bounds__(NW * 64) void splitkv_kernel(KernelArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KEYS = 32 * NW;
  constexpr int KP = DQK * 32 + kKPad;
  constexpr int VP = DV * 16 + 16;
  constexpr int DVP = DV * 16;
  constexpr int OP = DVP + 4;  // LDS pitch of the merged wave outputs (floats)
  // K and V tiles; after the key loop the same bytes hold one row block's wave outputs.
  constexpr int TILE_BYTES = KEYS * (KP + VP) * 2;
  constexpr int MERGE_BYTES = NW * NQB * 16 * OP * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vs = Ks + KEYS * KP;
  float (*wo)[NQB * 16 * OP] = reinterpret_cast<float (*)[NQB * 16 * OP]>(smem);
  __shared__ float wm[NW][NQB * 16], wl[NW][NQB * 16];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  Timeline tl(NW);
  tl.mark<0>();
  // Workgroups are dealt to the 8 XCDs round robin (workgroup i to XCD i % 8),
  // each XCD with its own L2.  Renumber so that every XCD gets a contiguous
  // range of (group, split) pairs: the position blocks of one unit, which
  // read the same K/V rows, then share them in one L2.
  // Every argument the first tile request depends on, asked for at once, so
  // that their loads leave in one batch and cost one round trip.
  const long long kv_stride = a.kv_stride;
  asm volatile("" : : "s"(kv_stride), "s"(a.k), "s"(a.v), "s"(a.nsplit), "s"(a.n_pos_blk), "s"(a.Hkv),
               "s"(a.m), "s"(a.Lq), "s"(a.Lkv), "s"(a.d), "s"(a.causal), "s"(a.window),
               "s"(a.tiles_per_split), "s"(a.div_nsplit.m), "s"(a.div_nsplit.s), "s"(a.div_npos.m),
               "s"(a.div_npos.s), "s"(a.div_hkv.m), "s"(a.div_hkv.s), "s"(a.nwg));
  // With two column halves the pair sharing a key range is adjacent, so it
  // runs on one XCD at the same time and K comes from HBM once.
  int lin = blockIdx.x;
  if ((a.nwg & 7) == 0) lin = (lin & 7) * (a.nwg >> 3) + (lin >> 3);
  const int half = NCOL == 2 ? (lin & 1) : 0;
  const int lsp = NCOL == 2 ? (lin >> 1) : lin;   // (group, split) index
  const int col0 = half * DV * 16;                  // first V/O column of this workgroup
  const int grp = fdiv(lsp, a.div_nsplit);  // unit * n_pos_blk + position block
  const int split = lsp - grp * a.nsplit;
  const int unit = fdiv(grp, a.div_npos);
  const int pblk = grp - unit * a.n_pos_blk;
  const int b = fdiv(unit, a.div_hkv), kvh = unit - b * a.Hkv;
  const int G = a.G, d = a.d;
  const int off = a.Lkv - a.Lq;
  const int q0 = pblk * a.m;
  const int m_eff = min(a.m, a.Lq - q0);
  const int nrows = m_eff * G;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (size_t)unit * kv_stride;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (size_t)unit * kv_stride;
  uint16_t* og = static_cast<uint16_t*>(a.out);

  // Key band of this block of positions, in tiles, and this split's share.
  const int pos_min = q0 + off, pos_max = q0 + m_eff - 1 + off;
  int key_lo = 0, key_hi = a.Lkv - 1;
  if (a.causal) key_hi = min(key_hi, pos_max);
  if (a.window > 0) {
    key_lo = max(0, pos_min - a.window + 1);
    if (!a.causal) key_hi = min(key_hi, pos_max + a.window - 1);
  }
  const int t0 = key_lo / KEYS + split * a.tiles_per_split;
  const int t1 = min(key_hi / KEYS + 1, t0 + a.tiles_per_split);
  // Staging registers for the next tile; with column halves (half-width V
  // tiles) a second set keeps two tiles in flight.
  constexpr bool TWO_AHEAD = NCOL == 2;
  using KTile = RowTile<KEYS, DQK * 4, KP, NT, STREAM ? kStreamLoad : 0>;
  using VTile = RowTile<KEYS, DV * 2, VP, NT, STREAM ? kStreamLoad : 0>;
  KTile kt, kt2;
  VTile vt, vt2;
  kt.init(d, tid);
  vt.init(d, tid, col0);
  if constexpr (TWO_AHEAD) {
    kt2.init(d, tid);
    vt2.init(d, tid, col0);
  }
  auto fetch_into = [&](KTile& ks, VTile& vs, bool k_part, int k0) {
    if (k_part) {
      if (RING) ks.load_ring(kg, k0, a.Lkv, d, a.ring_start, a.ring_slots, tid);
      else ks.load(kg, k0, a.Lkv, d);
    } else {
      if (RING) vs.load_ring(vg, k0, a.Lkv, d, a.ring_start, a.ring_slots, tid, col0);
      else vs.load(vg, k0, a.Lkv, d);
    }
    // Fused cache append: the appended keys are the last app_len keys, one
    // per query position, and come from the float32 rows.  The workgroup
    // whose position block holds query position i writes key app_pos + i to
    // its cache slot (K by the first column half only, V by each half for its
    // columns); no workgroup reads those cache slots.
    if (a.app_len > 0 && k0 < a.app_pos + a.app_len && k0 + KEYS > a.app_pos) {
      const size_t src = (size_t)unit * a.app_len * d;
      const int rs = RING ? a.ring_start : -1;
      if (k_part)
        ks.template substitute<T>(a.app_k + src, half == 0 ? const_cast<uint16_t*>(kg) : nullptr, k0, a.app_pos,
                                  a.app_len, q0, q0 + m_eff, d, tid, rs, a.ring_slots);
      else
        vs.template substitute<T>(a.app_v + src, const_cast<uint16_t*>(vg), k0, a.app_pos, a.app_len, q0,
                                  q0 + m_eff, d, tid, rs, a.ring_slots, col0);
    }
  };
  auto fetch_k = [&](int k0) { fetch_into(kt, vt, true, k0); };
  auto fetch_v = [&](int k0) { fetch_into(kt, vt, false, k0); };
  // The tiles of the range are visited in a rotated order that differs from
  // workgroup to workgroup, so that the workgroups do not all start on
  // addresses with the same alignment (which concentrates the first requests
  // on a few memory channels).  The softmax merge is order independent; the
  // order is a fixed function of the shape, so results stay reproducible.
  // The start is 5*(group, split index) modulo the largest power of two <=
  // ntile (a mask, no division, and always < ntile): the two column halves of
  // a key range take the same order, so they read each K tile together.
  const int ntile = max(t1 - t0, 0);
  const int rot = ntile > 0 ? (int)(((unsigned)lsp * 5u) & ((1u << (31 - __builtin_clz((unsigned)ntile))) - 1u)) : 0;
  auto tile_at = [&](int i) { const int r = i + rot; return t0 + (r >= ntile ? r - ntile : r); };
  if (ntile > 0) {
    fetch_k(tile_at(0) * KEYS);
    fetch_v(tile_at(0) * KEYS);
  }
  if constexpr (TWO_AHEAD) {
    if (ntile > 1) {
      fetch_into(kt2, vt2, true, tile_at(1) * KEYS);
      fetch_into(kt2, vt2, false, tile_at(1) * KEYS);
    }
  }

  // This lane's rows: column c16 of each 16-row block.
  u32x4 qf[NQB][DQK];
  int qpos[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = 16 * qb + c16;
    const bool rok = r < nrows;
    const int pl = fdiv(r, a.div_g), hr = r - pl * G;
    const size_t roff = (((size_t)b * a.Hq + kvh * G + hr) * a.Lq + (rok ? q0 + pl : 0)) * d;
    qpos[qb] = q0 + pl + off;
    load_q<DQK>(qf[qb], qg + roff, rok, d, g4);
  }
  tl.mark<1>();

  float m_e[NQB];
  f32x4 ls[NQB], o[NQB][DV];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_e[qb] = kNegInf;
    ls[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DV; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // This wave's 32 keys of the tile at k0: skipped when wholly outside the
  // band, unmasked when wholly inside it.
  auto compute = [&](int k0) {
    const int w0 = k0 + 32 * wave;
    if (w0 > key_hi || w0 + 31 < key_lo) return;
    bool full = w0 + 32 <= a.Lkv;
    if (a.causal) full = full && (w0 + 31 <= pos_min);
    if (a.window > 0) {
      full = full && (pos_max - w0 < a.window);
      if (!a.causal) full = full && (w0 + 31 - pos_min < a.window);
    }
    // With several row blocks, one copy of the step with a run-time mask
    // flag: separate full and masked copies leave the accumulators in
    // different registers on the two paths, merged by register moves on
    // every tile.
    if constexpr (NQB > 1)
      tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, true>(Ks, Vs, 32 * wave, k0, qf, qpos, m_e, ls, o, a, c16, g4,
                                                        !full);
    else if (full)
      tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, false>(Ks, Vs, 32 * wave, k0, qf, qpos, m_e, ls, o, a, c16, g4);
    else
      tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, true>(Ks, Vs, 32 * wave, k0, qf, qpos, m_e, ls, o, a, c16, g4);
  };
  if constexpr (TWO_AHEAD) {
    // Tiles alternate between the two register sets; each set is refilled
    // with the tile two ahead as soon as it is in LDS.
    for (int it = 0; it < ntile; it += 2) {
      __syncthreads();  // every wave is done with the previous tile
      kt.store(Ks, tid);
      if (it + 2 < ntile) fetch_into(kt, vt, true, tile_at(it + 2) * KEYS);
      vt.store(Vs, tid);
      if (it + 2 < ntile) fetch_into(kt, vt, false, tile_at(it + 2) * KEYS);
      __syncthreads();
      if (it == 0) tl.mark<2>();
      compute(tile_at(it) * KEYS);
      if (it + 1 >= ntile) break;
      __syncthreads();
      kt2.store(Ks, tid);
      if (it + 3 < ntile) fetch_into(kt2, vt2, true, tile_at(it + 3) * KEYS);
      vt2.store(Vs, tid);
      if (it + 3 < ntile) fetch_into(kt2, vt2, false, tile_at(it + 3) * KEYS);
      __syncthreads();
      compute(tile_at(it + 1) * KEYS);
    }
  } else {
    for (int it = 0; it < ntile; ++it) {
      const int k0 = tile_at(it) * KEYS;
      __syncthreads();  // every wave is done with the previous tile
      // Each half of the staging registers is refilled with the next tile as
      // soon as it is in LDS, so loads stay in flight while the other half is
      // written, and the next tile flies during this one.
      const bool more = it + 1 < ntile;
      const int kn = more ? tile_at(it + 1) * KEYS : 0;
      kt.store(Ks, tid);
      if (more) fetch_k(kn);
      vt.store(Vs, tid);
      if (more) fetch_v(kn);
      __syncthreads();
      if (it == 0) tl.mark<2>();
      const int w0 = k0 + 32 * wave;
      if (w0 > key_hi || w0 + 31 < key_lo) continue;
      bool full = w0 + 32 <= a.Lkv;
      if (a.causal) full = full && (w0 + 31 <= pos_min);
      if (a.window > 0) {
        full = full && (pos_max - w0 < a.window);
        if (!a.causal) full = full && (w0 + 31 - pos_min < a.window);
      }
      if constexpr (NQB > 1)  // one copy of the step, as in compute() above
        tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, true>(Ks, Vs, 32 * wave, k0, qf, qpos, m_e, ls, o, a, c16,
                                                          g4, !full);
      else if (full)
        tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, false>(Ks, Vs, 32 * wave, k0, qf, qpos, m_e, ls, o, a, c16,
                                                           g4);
      else
        tile_step<T, DQK, DV, NQB, KP, VP, SOFTCAP, true>(Ks, Vs, 32 * wave, k0, qf, qpos, m_e, ls, o, a, c16,
                                                          g4);
    }
  }

  tl.mark<3>();

  // ---- merge the wave states (fixed order) ------------------------------------
  // Every wave writes its (max, sum, unnormalised rows) of all row blocks to
  // LDS with 16-byte stores; after one barrier, thread -> float4 chunks
  // q = tid + NT*j of the [rows][DVP] output: row q / CPR, columns
  // 4*(q % CPR) .. +3, so a wave touches contiguous memory.
  constexpr int CPR = DVP / 4;
  constexpr int JN = (NQB * 16 * CPR + NT - 1) / NT;
  const int rstride = a.nrows;  // rows of a full block: partial layout stride
  // Partials: O rows [group][split][row] of NCOL*DVP floats (a column half
  // writes its DVP of them); (max, sum) [group][half][split][row].
  const int dvw = NCOL * DVP;
  const int pidx = (grp * a.nsplit + split) * rstride;
  const int pml = ((grp * NCOL + half) * a.nsplit + split) * rstride;
  const uint32_t o_bytes = (uint32_t)a.nwg * rstride * DVP * 4;
  const uint32_t ml_bytes = (uint32_t)a.nwg * rstride * 8;
  const auto rs_o = make_rsrc(a.ws_o, o_bytes);
  const auto rs_ml = make_rsrc(a.ws_ml, ml_bytes);
  __syncthreads();  // the tiles are no longer read
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    if (g4 == 0) {
      wm[wave][16 * qb + c16] = m_e[qb];
      wl[wave][16 * qb + c16] = ls[qb][0];
    }
#pragma unroll
    for (int db = 0; db < DV; ++db)
      *reinterpret_cast<f32x4*>(&wo[wave][(16 * qb + c16) * OP + 16 * db + 4 * g4]) = o[qb][db];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int q = tid + j * NT;
    const int r = q / CPR, c4 = q % CPR;
    if (q >= NQB * 16 * CPR || r >= nrows) continue;
    float M = kNegInf, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w][r]);
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(wm[w][r] - M);
        L += f * wl[w][r];
        const f32x4 x = *reinterpret_cast<const f32x4*>(&wo[w][r * OP + 4 * c4]);
        acc += f * x;
      }
    }
    if (a.nsplit == 1) {
      if (col0 + 4 * c4 < d) {
        const float inv = 1.0f / L;
        const int pr = fdiv(r, a.div_g);
        const size_t oo =
            (((size_t)b * a.Hq + kvh * G + (r - pr * G)) * a.Lq + q0 + pr) * d + col0 + 4 * c4;
        *reinterpret_cast<u32x2*>(og + oo) =
            u32x2{Elem<T>::pack2(acc[0] * inv, acc[1] * inv), Elem<T>::pack2(acc[2] * inv, acc[3] * inv)};
      }
    } else {
      // This split's partial, with device-coherent stores.
      st_dev16(rs_o, ((pidx + r) * dvw + col0 + 4 * c4) * 4, acc);
      if (c4 == 0) st_dev8(rs_ml, (pml + r) * 8, f32x2{M, L});
    }
  }
  tl.mark<4>();
  if (a.nsplit == 1) {
    tl.flush();
    return;
  }

  wait_vmem_done();
  __syncthreads();
  tl.mark<5>();
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(a.ws_cnt + grp * NCOL + half, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == (unsigned)(a.nsplit - 1)) ? 1 : 0;
  }
  __syncthreads();
  tl.mark<6>();
  if (!last_flag) {
    tl.flush();
    return;
  }

  // ---- last arrival: merge all splits in split order ---------------------------------
  // Online merge over groups of CHUNK splits (4, 8 or 16: the smallest that
  // holds every split when there are at most 16, so no load repeats a split);
  // every load of a group is issued before any of them is used.
  constexpr int JM = (16 * NQB * CPR + NT - 1) / NT;
  const int nch = nrows * CPR;
  const int base = grp * a.nsplit * rstride;                   // O rows of split 0
  const int base_ml = (grp * NCOL + half) * a.nsplit * rstride;  // (max, sum) of split 0
  auto merge_splits = [&](auto chunk_tag) {
    constexpr int CHUNK = decltype(chunk_tag)::value;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      const int q = tid + j * NT;
      if (q >= nch) continue;
      const int row = q / CPR, c4 = q % CPR;
      float Mg = kNegInf, Lg = 0.f;
      f32x4 og4 = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < a.nsplit; s0 += CHUNK) {
        f32x2 ml[CHUNK];
        f32x4 x[CHUNK];
#pragma unroll
        for (int jj = 0; jj < CHUNK; ++jj) {
          const int sp = min(s0 + jj, a.nsplit - 1);
          ml[jj] = ld_dev8(rs_ml, (base_ml + sp * rstride + row) * 8);
          x[jj] = ld_dev16(rs_o, ((base + sp * rstride + row) * dvw + col0 + 4 * c4) * 4);
        }
        float mc = Mg;
#pragma unroll
        for (int jj = 0; jj < CHUNK; ++jj)
          if (s0 + jj < a.nsplit) mc = fmaxf(mc, ml[jj][0]);
        // No branch here, so the compiler can keep all loads of a group in flight.
        const bool any = mc != kNegInf;
        const float fr = any ? fast_exp2(Mg - mc) : 1.f;  // 0 while nothing was merged yet
        Lg *= fr;
        og4 *= fr;
        Mg = any ? mc : Mg;
#pragma unroll
        for (int jj = 0; jj < CHUNK; ++jj) {
          const float f =
              (s0 + jj < a.nsplit && ml[jj][0] != kNegInf) ? fast_exp2(ml[jj][0] - Mg) : 0.f;
          Lg += f * ml[jj][1];
          og4 += f * x[jj];
        }
      }
      if (col0 + 4 * c4 < d) {
        const float inv = 1.0f / Lg;
        const int pr = fdiv(row, a.div_g);
        const size_t oo =
            (((size_t)b * a.Hq + kvh * G + (row - pr * G)) * a.Lq + q0 + pr) * d + col0 + 4 * c4;
        *reinterpret_cast<u32x2*>(og + oo) =
            u32x2{Elem<T>::pack2(og4[0] * inv, og4[1] * inv), Elem<T>::pack2(og4[2] * inv, og4[3] * inv)};
      }
    }
  };
  if (a.nsplit <= 4)
    merge_splits(std::integral_constant<int, 4>{});
  else if (a.nsplit <= 8)
    merge_splits(std::integral_constant<int, 8>{});
  else
    merge_splits(std::integral_constant<int, 16>{});
  if (tid == 0)
    __hip_atomic_store(a.ws_cnt + grp * NCOL + half, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  tl.mark<7>();
  tl.flush();
}

// ---------------------------------------------------------------------------
// Short-band kernel (encoder-sized sequences).
//
// One workgroup of 8 waves per (unit, block of 48 rows).  The block's key
// band, at most 768 keys, is cut into 8 contiguous wave ranges of up to three
// 32-key steps.  A wave reads only its own keys: its K fragments go straight
// from memory into registers (the A operand of S^T = K Q^T takes 8
// consecutive head-size elements of one key per lane: a piece of a row-major
// K row), and its V rows go into a private LDS region through direct
// global-to-LDS loads, from where the transposing LDS read builds V^T.  No
// tile is shared between waves, so the key loop has no barrier.
//
// With every score of its range in registers, a wave takes the row maximum
// once and one exponential per score (two passes over registers): no running
// maximum and no rescale.  The code is straight-line over three steps for
// every wave; steps past a wave's share have all keys masked (probability 0;
// the V rows they multiply are other keys' rows, or zeros past Lkv).  Row sums come from the matrix cores (all-ones A
// operand, the same 16-bit P as P.V).  The eight wave states then merge in
// LDS in wave order; once a wave's P.V products are done, its region holds
// its unnormalised rows (48 rows of DV*16 floats, padded by 4).
//
// Q.K^T contracts the head size in DQK 32-deep matrix-core steps (head size
// 72 padded to 96 with zeros).  A 16-deep product chained onto 32-deep ones
// through the accumulator was tried for 72 -> 80 and gave wrong results with
// this compiler (the chained product read an accumulator that was not yet
// written); every accumulator chain here uses one product shape.
// ---------------------------------------------------------------------------
template <typename T, int DQK, int DV, bool SOFTCAP>
__global__ __launch_bounds__(64 * kEncWaves) void encoder_kernel(KernelArgs a) {
  constexpr int NW = kEncWaves, NS = kEncSteps, NQB = kEncNqb;
  constexpr int VPITCH = DV * 16;           // elements of one staged V row
  constexpr int CPR = DV * 2;               // 16-byte chunks of one staged V row
  constexpr int VLOADS = 32 * CPR / 64;     // 64-lane direct-to-LDS loads per step
  // Floats of one output row in the merge: 16 bytes of padding put the 16
  // rows of one 16-lane group of a row-block store on distinct LDS banks
  // (unpadded, rows 4 apart shared banks: 4-way conflicts on every store).
  constexpr int OPITCH = DV * 16 + 4;
  constexpr int VELEMS = NS * 32 * VPITCH;    // elements of one wave's staged V rows
  constexpr int OELEMS = NQB * 16 * OPITCH * 2;  // the same region holding its output rows
  constexpr int REGION = VELEMS > OELEMS ? VELEMS : OELEMS;  // elements of one wave's region
  static_assert(DQK >= 1, "at least one 32-deep step");
  static_assert((32 * CPR) % 64 == 0, "a step's V rows are whole 64-lane loads");
  static_assert(REGION % 8 == 0, "wave regions stay 16-byte aligned");
  __shared__ __attribute__((aligned(16))) uint16_t sv[NW * REGION];
  __shared__ float wm[NW][NQB * 16], wl[NW][NQB * 16];
  __shared__ float wf[NW][NQB * 16];  // merge weight of each wave's rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int g4 = lane >> 4, c16 = lane & 15;
  Timeline tl(kEncWaves);
  tl.mark<0>();
  // Every argument the first loads depend on, asked for at once.
  const long long kv_stride = a.kv_stride;
  asm volatile("" : : "s"(kv_stride), "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.n_pos_blk), "s"(a.Hkv), "s"(a.Hq),
               "s"(a.G), "s"(a.m), "s"(a.Lq), "s"(a.Lkv), "s"(a.d), "s"(a.causal), "s"(a.window), "s"(a.div_g.m),
               "s"(a.div_g.s), "s"(a.div_npos.m), "s"(a.div_npos.s), "s"(a.div_hkv.m), "s"(a.div_hkv.s),
               "s"(a.nwg));
  // XCD-contiguous numbering, as in the other kernels: the position blocks
  // of one unit share its K/V rows in one L2.
  int lin = blockIdx.x;
  if ((a.nwg & 7) == 0) lin = (lin & 7) * (a.nwg >> 3) + (lin >> 3);
  const int unit = fdiv(lin, a.div_npos);
  const int pblk = lin - unit * a.n_pos_blk;
  const int b = fdiv(unit, a.div_hkv), kvh = unit - b * a.Hkv;
  const int G = a.G, d = a.d;
  const int off = a.Lkv - a.Lq;
  const int q0 = pblk * a.m;
  const int m_eff = min(a.m, a.Lq - q0);
  const int nrows = m_eff * G;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (size_t)unit * kv_stride;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (size_t)unit * kv_stride;
  uint16_t* og = static_cast<uint16_t*>(a.out);

  // Key band of the block, and this wave's share of its 32-key steps.
  const int pos_min = q0 + off, pos_max = q0 + m_eff - 1 + off;
  int key_lo = 0, key_hi = a.Lkv - 1;
  if (a.causal) key_hi = min(key_hi, pos_max);
  if (a.window > 0) {
    key_lo = max(0, pos_min - a.window + 1);
    if (!a.causal) key_hi = min(key_hi, pos_max + a.window - 1);
  }
  const int kb0 = key_lo & ~31;
  const int nsteps = (key_hi - kb0) / 32 + 1;  // at most NW * NS (the plan checks)
  const int spw = (nsteps + NW - 1) / NW;
  const int my = max(0, min(spw, nsteps - wave * spw));  // this wave's steps (wave-uniform)
  const int kw0 = kb0 + 32 * wave * spw;                  // this wave's first key

  // Keys at or past Lkv lie outside the descriptors' ranges and read as zero.
  const uint32_t unit_bytes = (uint32_t)a.Lkv * (uint32_t)d * 2u;
  const auto rs_k = make_rsrc(kg, unit_bytes);
  const auto rs_v = make_rsrc(vg, unit_bytes);

  // Q^T operands: lane column c16 is the row, lane group g4 holds head-size
  // elements 32t + 8g4 .. +7 of step t.
  u32x4 qf[NQB][DQK];
  int rlo[NQB], rspan[NQB];  // visible keys of this lane's row: [rlo, rlo + rspan]
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = 16 * qb + c16;
    const bool rok = r < nrows;
    const int pl = fdiv(r, a.div_g), hr = r - pl * G;
    const int pos = q0 + pl + off;
    int lo = 0, hi = a.Lkv - 1;
    if (a.causal) hi = min(hi, pos);
    if (a.window > 0) {
      lo = max(0, pos - a.window + 1);
      if (!a.causal) hi = min(hi, pos + a.window - 1);
    }
    rlo[qb] = lo;
    rspan[qb] = hi - lo;
    const uint16_t* qrow = qg + (((size_t)b * a.Hq + kvh * G + hr) * a.Lq + (rok ? q0 + pl : 0)) * d;
#pragma unroll
    for (int t = 0; t < DQK; ++t) {
      const int col = 32 * t + 8 * g4;
      qf[qb][t] = (rok && col < d) ? ldg16(qrow + col) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // K fragments of every step of this wave (registers) first, then its V rows
  // (LDS): the scores wait for K only, and V lands while they are computed.
  // Per-lane byte offsets are fixed; a step adds 32 rows through the
  // instruction's scalar offset.  All NS steps are loaded whatever the wave's
  // share (straight-line code, so the compiler counts the loads exactly);
  // steps past the share read keys of the next range or zeros past Lkv and
  // are never used.
  const uint32_t step_bytes = 32u * (uint32_t)d * 2u;
  u32x4 kf[NS][2][DQK];
  {
    uint32_t koff[2][DQK];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int t = 0; t < DQK; ++t) {
        const int col = 32 * t + 8 * g4;
        koff[hh][t] = col < d ? ((uint32_t)(kw0 + 16 * hh + c16) * (uint32_t)d + (uint32_t)col) * 2u : kOutOfRange;
      }
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int t = 0; t < DQK; ++t)
            kf[st][hh][t] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_k, (int)koff[hh][t], (int)(st * step_bytes), 0));
  }
  // (Keeps the scheduler from sinking the K loads below the V loads.)
  __builtin_amdgcn_sched_barrier(0);
  uint16_t* const myv = sv + wave * REGION;
  {
    uint32_t voff[VLOADS];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int n = 64 * i + lane;  // chunk n of a step's rows: row n / CPR, chunk n % CPR
      const int row = n / CPR, ch = n - row * CPR;
      voff[i] = ch * 8 < d ? ((uint32_t)(kw0 + row) * (uint32_t)d + (uint32_t)(ch * 8)) * 2u : kOutOfRange;
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < VLOADS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs_v, (__attribute__((address_space(3))) void*)(myv + st * 32 * VPITCH + i * 512), 16, (int)voff[i],
              (int)(st * step_bytes), 0, 0);
  }
  tl.mark<1>();

  // ---- scores S^T = K Q^T of every step ------------------------------------
  // Straight-line over all NS steps; steps past this wave's share are masked
  // out below.
  f32x4 s[NS][2][NQB];
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DQK; ++t) acc = Elem<T>::mfma(kf[st][hh][t], qf[qb][t], acc);
        s[st][hh][qb] = acc;
      }
  tl.mark<2>();

  // ---- mask: steps crossing a band edge or the end of the keys, and steps
  // past this wave's share (all keys) ------------------------------------------
  bool part[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int k0 = kw0 + 32 * st;
    bool full = k0 + 32 <= a.Lkv;
    if (a.causal) full = full && (k0 + 31 <= pos_min);
    if (a.window > 0) {
      full = full && (pos_max - k0 < a.window);
      if (!a.causal) full = full && (k0 + 31 - pos_min < a.window);
    }
    const bool mine = st < my;
    part[st] = !mine || !full;
    if (!mine) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) s[st][hh][qb] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
    } else if (part[st]) {
      // key j is visible to the row iff (unsigned)(j - lo) <= span
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int ub = k0 + 4 * g4 - rlo[qb];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((unsigned)(ub + 16 * hh + i) > (unsigned)rspan[qb]) s[st][hh][qb][i] = kNegInf;
      }
    }
  }

  // ---- row maxima over the whole range, then the probabilities --------------
  // The softcap is increasing, so the maximum of the capped scores is the
  // capped maximum score (same formula, so the maximum maps to exactly 2^0).
  float m_e[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float mx = kNegInf;
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[st][hh][qb][i]);
    mx = col_max(mx);
    if (SOFTCAP)
      m_e[qb] = (mx == kNegInf) ? kNegInf
                                : __builtin_fmaf(fast_rcp(fast_exp2(mx * a.gamma) + 1.0f), -2.0f * a.c2, a.c2);
    else
      m_e[qb] = mx * a.alpha;
  }
  const u32x4 ones = {OnesOperand<T>::kPair, OnesOperand<T>::kPair, OnesOperand<T>::kPair, OnesOperand<T>::kPair};
  u32x4 pk[NS][NQB];
  f32x4 ls[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    ls[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float mref = (m_e[qb] == kNegInf) ? 0.f : m_e[qb];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float p[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = s[st][hh][qb][i];
          float pv;
          if (SOFTCAP) {
            // c*tanh(u) = c - 2c/(exp(2u)+1), in base-2 exponent units.
            const float r = fast_rcp(fast_exp2(x * a.gamma) + 1.0f);
            pv = fast_exp2(__builtin_fmaf(r, -2.0f * a.c2, a.c2 - mref));
            if (part[st] && x == kNegInf) pv = 0.f;
          } else {
            pv = fast_exp2(__builtin_fmaf(x, a.alpha, -mref));
          }
          p[hh * 4 + i] = pv;
        }
      pk[st][qb] = u32x4{Elem<T>::pack2(p[0], p[1]), Elem<T>::pack2(p[2], p[3]), Elem<T>::pack2(p[4], p[5]),
                         Elem<T>::pack2(p[6], p[7])};
      ls[qb] = Elem<T>::mfma(ones, pk[st][qb], ls[qb]);
    }
  }
  tl.mark<3>();

  // ---- O^T = V^T P^T over the range ------------------------------------------
  // Transposed reads as in the other kernels: lane s of a 16-lane group points
  // at key row 4*g4 + s/4 (and +16), columns 16*db + 4*(s%4).
  f32x4 o[NQB][DV];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int db = 0; db < DV; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const uint16_t* v0 = myv + (32 * st + 4 * g4 + (c16 >> 2)) * VPITCH + 4 * (c16 & 3);
#pragma unroll
    for (int db = 0; db < DV; ++db) {
      const u32x2 lo = lds_read_tr4(v0 + 16 * db);
      const u32x2 hi = lds_read_tr4(v0 + 16 * VPITCH + 16 * db);
      const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) o[qb][db] = Elem<T>::mfma(vf, pk[st][qb], o[qb][db]);
    }
  }
  tl.mark<4>();

  // ---- merge the eight wave states in wave order -----------------------------
  // The products above consumed this wave's V reads, so its region is free.
  float* wo = reinterpret_cast<float*>(myv);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    if (g4 == 0) {
      wm[wave][16 * qb + c16] = m_e[qb];
      wl[wave][16 * qb + c16] = ls[qb][0];
    }
#pragma unroll
    for (int db = 0; db < DV; ++db)
      *reinterpret_cast<f32x4*>(&wo[(16 * qb + c16) * OPITCH + 16 * db + 4 * g4]) = o[qb][db];
  }
  __syncthreads();
  tl.mark<5>();
  // Weight of wave w's row r: 2^(m_w - M) / L with M the row's maximum over
  // the waves and L = sum_w 2^(m_w - M) l_w (each sum in wave order); one
  // thread per (row, wave).
  static_assert(NQB * 16 * NW <= 64 * NW, "one thread per (row, wave)");
  if (tid < NQB * 16 * NW) {
    const int r = tid / NW, w = tid - r * NW;
    float M = kNegInf;
#pragma unroll
    for (int u = 0; u < NW; ++u) M = fmaxf(M, wm[u][r]);
    float L = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) L += (wm[u][r] == kNegInf ? 0.f : fast_exp2(wm[u][r] - M)) * wl[u][r];
    wf[w][r] = (wm[w][r] == kNegInf) ? 0.f : fast_exp2(wm[w][r] - M) / L;
  }
  __syncthreads();
  tl.mark<6>();
  constexpr int C4 = DV * 4;  // float4 chunks of one output row
  constexpr int JN = (NQB * 16 * C4 + 64 * NW - 1) / (64 * NW);
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int q = tid + j * 64 * NW;
    const int r = q / C4, c4 = q - r * C4;
    if (q >= NQB * 16 * C4 || r >= nrows || 4 * c4 >= d) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w)
      acc += wf[w][r] * *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(sv + w * REGION) + r * OPITCH +
                                                      4 * c4);
    const int pr = fdiv(r, a.div_g);
    const size_t oo = (((size_t)b * a.Hq + kvh * G + (r - pr * G)) * a.Lq + q0 + pr) * d + 4 * c4;
    *reinterpret_cast<u32x2*>(og + oo) = u32x2{Elem<T>::pack2(acc[0], acc[1]), Elem<T>::pack2(acc[2], acc[3])};
  }
  tl.mark<7>();
  tl.flush();
}

__global__ void zero_kernel(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host-side dispatch over the instantiated shapes.
// ---------------------------------------------------------------------------
// Streaming (non-temporal) K/V loads when each unit has one position block
// (no workgroup re-reads another's rows; see kStreamLoad).
template <typename T, int DQK, int DV, int NQB, bool SOFTCAP, int NCOL = 1, int NW = kSplitWaves>
static void launch_split(const dim3& grid, const KernelArgs& args, hipStream_t st) {
  const dim3 block(64 * NW);
  if (NQB == 1 && args.ring_start >= 0)  // ring caches: decode only, one position block
    hipLaunchKernelGGL((splitkv_kernel<T, DQK, DV, 1, NW, SOFTCAP, true, NCOL, true>), grid, block, 0, st, args);
  else if (args.n_pos_blk == 1)
    hipLaunchKernelGGL((splitkv_kernel<T, DQK, DV, NQB, NW, SOFTCAP, false, NCOL, true>), grid, block, 0, st, args);
  else
    hipLaunchKernelGGL((splitkv_kernel<T, DQK, DV, NQB, NW, SOFTCAP, false, NCOL, false>), grid, block, 0, st,
                       args);
}

template <typename T, int DQK, int DV, bool SOFTCAP>
static hipError_t launch_typed(const Plan& plan, const KernelArgs& args, hipStream_t st) {
  const dim3 grid((unsigned)plan.workgroups);
  if (plan.path == kPathSplit) {
    if (plan.nwaves == kSplitWavesWide) {
      // Eight waves over 256-key tiles, full width, one 16-row block (long
      // decode ranges).
      if (plan.ncol != 1 || plan.nqb != 1) return hipErrorInvalidValue;
      launch_split<T, DQK, DV, 1, SOFTCAP, 1, kSplitWavesWide>(grid, args, st);
      return hipGetLastError();
    }
    if (plan.ncol == 2) {
      // Two column halves: each workgroup computes half of P.V's 16-column blocks.
      if constexpr (DV == 8) {
        launch_split<T, DQK, 4, 1, SOFTCAP, 2>(grid, args, st);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    }
    switch (plan.nqb) {
      case 1: launch_split<T, DQK, DV, 1, SOFTCAP>(grid, args, st); break;
      case 2: launch_split<T, DQK, DV, 2, SOFTCAP>(grid, args, st); break;
      case 3:
        if constexpr (DV <= kSplitWideMaxDv) launch_split<T, DQK, DV, 3, SOFTCAP>(grid, args, st);
        else return hipErrorInvalidValue;
        break;
      case 4:
        if constexpr (DV <= kSplitWideMaxDv) launch_split<T, DQK, DV, 4, SOFTCAP>(grid, args, st);
        else return hipErrorInvalidValue;
        break;
      default: return hipErrorInvalidValue;
    }
  } else if (args.d == 128) {
    // Fixed softmax reference: bf16 probabilities and a softcap small enough
    // that every exponent stays in range (c * log2(e) <= 83).
    if constexpr (SOFTCAP && __is_same(T, __bf16)) {
      if (args.c2 <= 83.0f) {
        hipLaunchKernelGGL((prefill_pipe4_kernel<T, true, true>), grid, dim3(64 * kPipe4Waves), 0, st, args);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((prefill_pipe4_kernel<T, SOFTCAP, false>), grid, dim3(64 * kPipe4Waves), 0, st, args);
  } else {
    if constexpr (DQK == 4)  // head sizes 104-120: one 16-row block per wave
      hipLaunchKernelGGL((prefill_kernel<T, DQK, DV, kPrefillNqbWide, kPrefillWaves, SOFTCAP>), grid,
                         dim3(64 * kPrefillWaves), 0, st, args);
    else
      hipLaunchKernelGGL((prefill_kernel<T, DQK, DV, kPrefillNqb, kPrefillWaves, SOFTCAP>), grid,
                         dim3(64 * kPrefillWaves), 0, st, args);
  }
  return hipGetLastError();
}

template <typename T, bool SOFTCAP>
static hipError_t launch_short(const Plan& plan, const KernelArgs& args, hipStream_t st) {
  const dim3 grid((unsigned)plan.workgroups), block(64 * kEncWaves);
  if (args.d > 80 && args.d <= 96)
    hipLaunchKernelGGL((encoder_kernel<T, 3, 6, SOFTCAP>), grid, block, 0, st, args);
  else if (args.d > 64)
    hipLaunchKernelGGL((encoder_kernel<T, 3, 5, SOFTCAP>), grid, block, 0, st, args);
  else if (args.d > 48)
    hipLaunchKernelGGL((encoder_kernel<T, 2, 4, SOFTCAP>), grid, block, 0, st, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, bool SOFTCAP>
static hipError_t launch_dims(const Plan& plan, const KernelArgs& args, hipStream_t st) {
  if (plan.path == kPathShort) return launch_short<T, SOFTCAP>(plan, args, st);
  switch (plan.dqk * 16 + plan.dv) {
    case 1 * 16 + 2: return launch_typed<T, 1, 2, SOFTCAP>(plan, args, st);
    case 2 * 16 + 4: return launch_typed<T, 2, 4, SOFTCAP>(plan, args, st);
    case 3 * 16 + 5: return launch_typed<T, 3, 5, SOFTCAP>(plan, args, st);
    case 3 * 16 + 6: return launch_typed<T, 3, 6, SOFTCAP>(plan, args, st);
    case 4 * 16 + 8: return launch_typed<T, 4, 8, SOFTCAP>(plan, args, st);
    default: return hipErrorInvalidValue;
  }
}

int launch(const Plan& plan, const KernelArgs& args, int dtype, bool softcap, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == 0)
    return softcap ? launch_dims<__bf16, true>(plan, args, st) : launch_dims<__bf16, false>(plan, args, st);
  return softcap ? launch_dims<_Float16, true>(plan, args, st) : launch_dims<_Float16, false>(plan, args, st);
}

int launch_zero(void* p, size_t words, void* stream) {
  if (words == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((words + 255) / 256);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace mgqa

#ifdef MGQA_TIMELINE
// Timeline build only: the wave records (include/mgqa_timeline.h).
static int timeline_address(void** ptr) {
  *ptr = nullptr;
  if (hipGetSymbolAddress(ptr, HIP_SYMBOL(mgqa::g_timeline)) != hipSuccess || *ptr == nullptr) return MGQA_ERR_HIP;
  return MGQA_OK;
}

extern "C" int attn_timeline_layout(int* events, int* max_waves) {
  if (events == nullptr || max_waves == nullptr) return MGQA_ERR_NULL;
  *events = mgqa::kTlEvents;
  *max_waves = mgqa::kTlMaxWaves;
  return MGQA_OK;
}

extern "C" int attn_timeline_clear(void* stream) {
  void* ptr;
  const int err = timeline_address(&ptr);
  if (err != MGQA_OK) return err;
  const size_t words32 = sizeof(mgqa::g_timeline) / 4;
  return mgqa::launch_zero(ptr, words32, stream) == hipSuccess ? MGQA_OK : MGQA_ERR_HIP;
}

extern "C" int attn_timeline_read(unsigned long long* host, size_t words) {
  if (host == nullptr) return MGQA_ERR_NULL;
  if (words > sizeof(mgqa::g_timeline) / 8) return MGQA_ERR_RANGE;
  void* ptr;
  const int err = timeline_address(&ptr);
  if (err != MGQA_OK) return err;
  if (hipDeviceSynchronize() != hipSuccess) return MGQA_ERR_HIP;
  if (words > 0 && hipMemcpy(host, ptr, words * 8, hipMemcpyDeviceToHost) != hipSuccess) return MGQA_ERR_HIP;
  return MGQA_OK;
}
#endif
