// KV-cache update at a position (TensorTonic, "KV Cache Update at a
// Position"): slots position .. position+L-1 of every (batch, head) row of the
// key and value caches receive the new float32 vectors, converted to the cache
// element type with round-to-nearest-even; nothing else is written.  One
// thread per element of the new vectors; both tensors' element offsets come
// from the layout (0: [B][S][H][D] / [B][L][H][D], 1: [B][H][S][D] /
// [B][H][L][D]).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgqa.h"
#include "mgqa_internal.h"

namespace mgqa {

template <typename TC>
__device__ __forceinline__ TC from_f32(float x) { return (TC)x; }

template <typename TC>
__global__ __launch_bounds__(256) void append_kernel(TC* kc, TC* vc, const float* nk, const float* nv,
                                                     int B, int S, int H, int D, int L, int position,
                                                     int layout, int* length_out) {
  const long long n = (long long)B * L * H * D;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0 && length_out) *length_out = position + L;
  if (i >= n) return;
  const int dd = (int)(i % D);
  long long rest = i / D;
  long long src, dst;
  if (layout == 0) {  // new [B][L][H][D] -> cache [B][S][H][D]
    const int h = (int)(rest % H);
    rest /= H;
    const int l = (int)(rest % L);
    const int b = (int)(rest / L);
    src = i;
    dst = (((long long)b * S + position + l) * H + h) * D + dd;
  } else {  // new [B][H][L][D] -> cache [B][H][S][D]
    const int l = (int)(rest % L);
    rest /= L;
    const int h = (int)(rest % H);
    const int b = (int)(rest / H);
    src = i;
    dst = (((long long)b * H + h) * S + position + l) * D + dd;
  }
  kc[dst] = from_f32<TC>(nk[src]);
  vc[dst] = from_f32<TC>(nv[src]);
}

int launch_append(void* kc, void* vc, const float* nk, const float* nv, int B, int S, int H, int D,
                  int L, int position, int cache_dtype, int layout, int* length_out, void* stream) {
  const long long n = (long long)B * L * H * D;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cache_dtype == MGQA_F32)
    hipLaunchKernelGGL(append_kernel<float>, dim3(blocks), dim3(256), 0, st, static_cast<float*>(kc),
                       static_cast<float*>(vc), nk, nv, B, S, H, D, L, position, layout, length_out);
  else if (cache_dtype == MGQA_BF16)
    hipLaunchKernelGGL(append_kernel<__bf16>, dim3(blocks), dim3(256), 0, st, static_cast<__bf16*>(kc),
                       static_cast<__bf16*>(vc), nk, nv, B, S, H, D, L, position, layout, length_out);
  else
    hipLaunchKernelGGL(append_kernel<_Float16>, dim3(blocks), dim3(256), 0, st,
                       static_cast<_Float16*>(kc), static_cast<_Float16*>(vc), nk, nv, B, S, H, D, L,
                       position, layout, length_out);
  return hipGetLastError();
}

}  // namespace mgqa
