// Throughput probes for gfx950 (libmgqa_probe.so, include/mgqa_probe.h):
// the matrix-core, transcendental and plain vector rates, how they mix in
// one step of the head-size-128 prefill, and the streaming read rate of
// device memory.  A measurement tool, separate from the attention library.
#include "mgqa_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgqa.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// An empty instruction that takes and returns v: the compiler cannot look
// through it, so a chain of operations on v is never folded.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

// Scheduling groups (the masks of __builtin_amdgcn_sched_group_barrier).
constexpr int kGroupValu = 0x002;
constexpr int kGroupMfma = 0x008;

template <int KIND>
__global__ __launch_bounds__(1024) void probe_alu_kernel(int iters, unsigned* sink) {
  const int tid = threadIdx.x, lane = tid & 63;
  // Matrix operands: 2^-6 in every element (each product adds 2^-7 to each
  // accumulator element, far from overflow for any practical iteration count).
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.015625f);
    b[i] = (__bf16)(0.015625f);
  }
  f32x4 acc[18];
  for (int c = 0; c < 18; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float y[16];
  for (int c = 0; c < 16; ++c) y[c] = 0.25f + 0.03125f * c + 0.0001f * lane;

  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == PROBE_MFMA || KIND == PROBE_MFMA_EXP || KIND == PROBE_MFMA_MUL) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = mfma(a, b, acc[c]);
    }
    if constexpr (KIND == PROBE_EXP || KIND == PROBE_MFMA_EXP) {
      // y <- 2^-y stays in [0.5, 1] for y in [0, 1].
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        y[c] = __builtin_amdgcn_exp2f(-y[c]);
        pin(y[c]);
      }
    }
    if constexpr (KIND == PROBE_RCP) {
      // y <- 1/y alternates between two values.
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        y[c] = __builtin_amdgcn_rcpf(y[c]);
        pin(y[c]);
      }
    }
    if constexpr (KIND == PROBE_MUL || KIND == PROBE_MFMA_MUL) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        y[c] = y[c] * 0.99993896484375f;
        pin(y[c]);
      }
    }
    if constexpr (KIND == PROBE_MFMA_EXP || KIND == PROBE_MFMA_MUL) {
      // One matrix product, then one vector operation, eight times.
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(kGroupMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kGroupValu, 1, 0);
      }
    }
    if constexpr (KIND == PROBE_STEP_MFMA || KIND == PROBE_STEP_BOTH) {
      // 32 products into 16 accumulators (scores and P.V) and 2 more (row sums).
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = mfma(a, b, acc[c]);
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = mfma(a, b, acc[c]);
      acc[16] = mfma(a, b, acc[16]);
      acc[17] = mfma(a, b, acc[17]);
    }
    if constexpr (KIND == PROBE_STEP_VEC || KIND == PROBE_STEP_BOTH) {
      // 16 softcapped probabilities per lane: e = 2^(s g), r = 1/(e + 1),
      // p = 2^(r c1 + c0); p feeds the next iteration (it stays in [0.7, 1.5]).
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float e = __builtin_amdgcn_exp2f(y[c] * 0.0408f);
        const float r = __builtin_amdgcn_rcpf(e + 1.0f);
        y[c] = __builtin_amdgcn_exp2f(__builtin_fmaf(r, -1.0f, 0.5f));
        pin(y[c]);
      }
    }
    if constexpr (KIND == PROBE_STEP_BOTH) {
      // The prefill kernel's interleave: one matrix product per three vector
      // operations.
#pragma unroll
      for (int g = 0; g < 34; ++g) {
        __builtin_amdgcn_sched_group_barrier(kGroupMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kGroupValu, 3, 0);
      }
    }
    if constexpr (KIND >= PROBE_STEP_MFMA) __syncthreads();
  }

  float s = 0.f;
  for (int c = 0; c < 18; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  for (int c = 0; c < 16; ++c) s += y[c];
  sink[(size_t)blockIdx.x * blockDim.x + tid] = __builtin_bit_cast(uint32_t, s);
}

// A 16-byte load, plain or non-temporal (the nt bit: kept in the caches
// only briefly).
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* src, size_t n, unsigned* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = x0, x2 = x0, x3 = x0;
  // Four independent loads in flight per thread.
  for (; i + 3 * stride < n; i += 4 * stride) {
    x0 ^= load16<NT>(src + i);
    x1 ^= load16<NT>(src + i + stride);
    x2 ^= load16<NT>(src + i + 2 * stride);
    x3 ^= load16<NT>(src + i + 3 * stride);
  }
  for (; i < n; i += stride) x0 ^= load16<NT>(src + i);
  const u32x4 x = x0 ^ x1 ^ x2 ^ x3;
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

template <int KIND>
hipError_t launch_alu(int workgroups, int waves, int iters, unsigned* sink, hipStream_t st) {
  hipLaunchKernelGGL(probe_alu_kernel<KIND>, dim3((unsigned)workgroups), dim3((unsigned)(64 * waves)), 0, st,
                     iters, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" int probe_alu(int kind, int workgroups, int waves, int iters, unsigned* sink, void* stream) {
  if (!sink) return MGQA_ERR_NULL;
  if (workgroups < 1 || waves < 1 || waves > 16 || iters < 1) return MGQA_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kind) {
    case PROBE_MFMA: e = launch_alu<PROBE_MFMA>(workgroups, waves, iters, sink, st); break;
    case PROBE_EXP: e = launch_alu<PROBE_EXP>(workgroups, waves, iters, sink, st); break;
    case PROBE_RCP: e = launch_alu<PROBE_RCP>(workgroups, waves, iters, sink, st); break;
    case PROBE_MUL: e = launch_alu<PROBE_MUL>(workgroups, waves, iters, sink, st); break;
    case PROBE_MFMA_EXP: e = launch_alu<PROBE_MFMA_EXP>(workgroups, waves, iters, sink, st); break;
    case PROBE_MFMA_MUL: e = launch_alu<PROBE_MFMA_MUL>(workgroups, waves, iters, sink, st); break;
    case PROBE_STEP_MFMA: e = launch_alu<PROBE_STEP_MFMA>(workgroups, waves, iters, sink, st); break;
    case PROBE_STEP_VEC: e = launch_alu<PROBE_STEP_VEC>(workgroups, waves, iters, sink, st); break;
    case PROBE_STEP_BOTH: e = launch_alu<PROBE_STEP_BOTH>(workgroups, waves, iters, sink, st); break;
    default: return MGQA_ERR_SHAPE;
  }
  return e == hipSuccess ? MGQA_OK : MGQA_ERR_HIP;
}

extern "C" int probe_read(const void* src, size_t bytes, int workgroups, int nontemporal, unsigned* sink,
                          void* stream) {
  if (!src || !sink) return MGQA_ERR_NULL;
  if (workgroups < 1 || bytes % 16 != 0 || (nontemporal != 0 && nontemporal != 1)) return MGQA_ERR_SHAPE;
  const dim3 grid((unsigned)workgroups), block(256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(probe_read_kernel<true>, grid, block, 0, st, static_cast<const u32x4*>(src), bytes / 16, sink);
  else
    hipLaunchKernelGGL(probe_read_kernel<false>, grid, block, 0, st, static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MGQA_OK : MGQA_ERR_HIP;
}
