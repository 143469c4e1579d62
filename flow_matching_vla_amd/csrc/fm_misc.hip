// Small kernels of the denoise loop: action/state in-projection (with the row statistics
// that the first modulated norm reads), conversions, and the bind-time copies of prefix
// K/V into the library's pool.
#include "fm_common.h"
#include "fm_kernels.h"

namespace fm {

// One workgroup (256 threads) per h row. Columns n = tid + 256 j; wave w of pass j covers
// statistic slot 4 j + w (64 columns), reduced across the wave with pairwise merges.
template <typename T>
__global__ void __launch_bounds__(256) k_inproj(InProjArgs a) {
  const int hr = blockIdx.x;
  const int per = a.st + a.Ha;
  const int b = hr / per, t = hr % per;
  const int lane = threadIdx.x & 63;
  for (int n0 = 0; n0 < a.D; n0 += 256) {
    const int n = n0 + threadIdx.x;
    float v = 0.f;
    if (n < a.D) {
      if (t < a.st) {
        v = a.state_tok[(long)(b * a.st + t) * a.D + n];
      } else {
        const float* xr = a.x + (long)(b * a.Ha + t - a.st) * a.da;
        const T* wr = (const T*)a.w + (long)n * a.da;
        float acc = 0.f;
        for (int k = 0; k < a.da; ++k) acc += xr[k] * to_f32(wr[k]);
        v = acc + a.b[n] + (a.tb ? a.tb[n] : 0.f);
      }
      a.h[(long)hr * a.D + n] = v;
    }
    if (a.stats) {
      float mean = v, m2 = 0.f, cnt = 1.f;
      for (int off = 1; off < 64; off <<= 1) {
        const float mb = __shfl_xor(mean, off, 64);
        const float qb = __shfl_xor(m2, off, 64);
        const float tot = 2.f * cnt;
        const float d = mb - mean;
        mean += d * 0.5f;
        m2 += qb + d * d * (cnt * cnt / tot);
        cnt = tot;
      }
      const int slot = (n0 + (threadIdx.x & ~63)) / kStatCols;
      if (lane == 0 && n0 + (threadIdx.x & ~63) < a.D) a.stats[(long)slot * a.stats_ld + hr] = make_float2(mean, m2);
    }
  }
}

hipError_t inproj_launch(const InProjArgs& a, int elem, hipStream_t s) {
  const int rows = a.B * (a.st + a.Ha);
  if (rows == 0) return hipSuccess;
  if (elem == ET_BF16) hipLaunchKernelGGL(k_inproj<bf16>, dim3(rows), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_inproj<float>, dim3(rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
__global__ void k_to_f32(float* dst, const T* src, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = to_f32(src[i]);
}
template <typename T>
__global__ void k_from_f32(T* dst, const float* src, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = from_f32<T>(src[i]);
}
__global__ void k_fill(float* dst, float v, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) dst[i] = v;
}

static int grid_for(long n) { long g = (n + 255) / 256; return (int)(g < 2048 ? (g > 0 ? g : 1) : 2048); }

hipError_t convert_to_f32(float* dst, const void* src, long n, int elem, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (elem == ET_BF16) hipLaunchKernelGGL(k_to_f32<bf16>, dim3(grid_for(n)), dim3(256), 0, s, dst, (const bf16*)src, n);
  else hipLaunchKernelGGL(k_to_f32<float>, dim3(grid_for(n)), dim3(256), 0, s, dst, (const float*)src, n);
  return hipGetLastError();
}
hipError_t convert_from_f32(void* dst, const float* src, long n, int elem, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (elem == ET_BF16) hipLaunchKernelGGL(k_from_f32<bf16>, dim3(grid_for(n)), dim3(256), 0, s, (bf16*)dst, src, n);
  else hipLaunchKernelGGL(k_from_f32<float>, dim3(grid_for(n)), dim3(256), 0, s, (float*)dst, src, n);
  return hipGetLastError();
}
hipError_t fill_f32(float* dst, float v, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill, dim3(grid_for(n)), dim3(256), 0, s, dst, v, n);
  return hipGetLastError();
}

// pool[b*pool_bs + j*dh + d'] = src[(b*P + j)*dh + perm(d')], perm interleaving RoPE pairs.
template <typename T>
__global__ void k_prefix_k(T* pool, long pool_bs, const T* src, int B, int P, int dh, int rope) {
  const long n = (long)B * P * dh;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int dp = (int)(i % dh);
    const long row = i / dh;
    const int b = (int)(row / P), j = (int)(row % P);
    const int d = rope ? ((dp & 1) ? dp / 2 + dh / 2 : dp / 2) : dp;
    pool[(long)b * pool_bs + (long)j * dh + dp] = src[row * dh + d];
  }
}
// pool[b*pool_bs + d*cap + j] = src[(b*P + j)*dh + d]
template <typename T>
__global__ void k_prefix_vt(T* pool, long pool_bs, int cap, const T* src, int B, int P, int dh) {
  const long n = (long)B * P * dh;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int j = (int)(i % P);
    const long r = i / P;
    const int d = (int)(r % dh), b = (int)(r / dh);
    pool[(long)b * pool_bs + (long)d * cap + j] = src[((long)b * P + j) * dh + d];
  }
}

hipError_t prefix_k_copy(void* pool, long pool_bs, const void* src, int B, int P, int dh, int rope, int elem,
                         hipStream_t s) {
  const long n = (long)B * P * dh;
  if (n <= 0) return hipSuccess;
  if (elem == ET_BF16)
    hipLaunchKernelGGL(k_prefix_k<bf16>, dim3(grid_for(n)), dim3(256), 0, s, (bf16*)pool, pool_bs, (const bf16*)src, B, P, dh, rope);
  else
    hipLaunchKernelGGL(k_prefix_k<float>, dim3(grid_for(n)), dim3(256), 0, s, (float*)pool, pool_bs, (const float*)src, B, P, dh, rope);
  return hipGetLastError();
}

hipError_t prefix_v_copy_t(void* pool, long pool_bs, int cap, const void* src, int B, int P, int dh, int elem,
                           hipStream_t s) {
  const long n = (long)B * P * dh;
  if (n <= 0) return hipSuccess;
  if (elem == ET_BF16)
    hipLaunchKernelGGL(k_prefix_vt<bf16>, dim3(grid_for(n)), dim3(256), 0, s, (bf16*)pool, pool_bs, cap, (const bf16*)src, B, P, dh);
  else
    hipLaunchKernelGGL(k_prefix_vt<float>, dim3(grid_for(n)), dim3(256), 0, s, (float*)pool, pool_bs, cap, (const float*)src, B, P, dh);
  return hipGetLastError();
}

}  // namespace fm
