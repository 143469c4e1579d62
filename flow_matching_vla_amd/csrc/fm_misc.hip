// Small kernels of the denoise loop: action/state in-projection (with the row statistics
// that the first modulated norm reads), conversions, and the bind-time copies of prefix
// K/V into the library's pool.
#include "fm_common.h"
#include "fm_kernels.h"

namespace fm {

// Workgroup = 64 h rows x 64 columns. The columns' weight rows and the rows' inputs are
// staged in LDS with every global load issued up front; thread (row r, 16-column group g)
// computes 16 outputs, stores them, and merges (mean, M2) of each kStatCols-column slot
// across the lanes of the row that share it.
constexpr int kInMaxK = 64;
template <typename T>
__global__ void __launch_bounds__(256) k_inproj(InProjArgs a) {
  __shared__ float sw[64][kInMaxK + 1];
  __shared__ float sx[64][kInMaxK + 1];
  const int per = a.st + a.Ha;
  const int rows = a.B * per;
  const int n0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  constexpr int LPT = 64 * kInMaxK / 256;
  float wv[LPT], xv[LPT];
  // unconditional loads from clamped indices; entries with k >= da are never read and
  // state-token rows ignore x
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    const int idx = tid + q * 256;
    const int rr = idx / kInMaxK, k = min(idx % kInMaxK, a.da - 1);
    wv[q] = to_f32(((const T*)a.w)[(long)(n0 + rr) * a.da + k]);
    const int hr = min(r0 + rr, rows - 1);
    const int b = hr / per, t = max(hr % per - a.st, 0);
    xv[q] = a.x[(long)(b * a.Ha + t) * a.da + k];
  }
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    const int idx = tid + q * 256;
    sw[idx / kInMaxK][idx % kInMaxK] = wv[q];
    sx[idx / kInMaxK][idx % kInMaxK] = xv[q];
  }
  const int r = tid / 4, g = tid % 4;
  const int hr = r0 + r;
  const bool rok = hr < rows;
  const int b = rok ? hr / per : 0, t = rok ? hr % per : 0;
  float bias[16], st[16], hsc[16];
  const int tst = min(t, a.st > 0 ? a.st - 1 : 0);
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    // unconditional loads; absent optional vectors read as zeros
    const int n = n0 + g * 16 + c;   // D is a multiple of 64: always in range
    const f32x4 bv = *(const f32x4*)(a.b + n);
    const f32x4 tv = *(const f32x4*)(a.tb + n);
    const f32x4 sv = *(const f32x4*)(a.hscale + n);
    const f32x4 stv = *(const f32x4*)(a.state_tok + (long)(b * a.st + tst) * a.D + n);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bias[c + j] = bv[j] + tv[j];
      hsc[c + j] = sv[j];
      st[c + j] = stv[j];
    }
  }
  __syncthreads();
  float y[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) y[c] = 0.f;
  for (int k = 0; k < a.da; ++k) {
    const float xk = sx[r][k];
#pragma unroll
    for (int c = 0; c < 16; ++c) y[c] += xk * sw[g * 16 + c][k];
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) y[c] = (rok && t < a.st) ? st[c] : y[c] + bias[c];
  if (rok && n0 + g * 16 < a.D) {
    float* hp = a.h + (long)hr * a.D + n0 + g * 16;
#pragma unroll
    for (int c = 0; c < 16; c += 4) *(f32x4*)(hp + c) = f32x4{y[c], y[c + 1], y[c + 2], y[c + 3]};
    if (a.hs) {
      T* hq = (T*)a.hs + (long)hr * a.D + n0 + g * 16;
      if constexpr (sizeof(T) == 2) {   // two 16-byte stores (the row piece is 32-byte aligned)
#pragma unroll
        for (int c = 0; c < 16; c += 8) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (bf16)(y[c + e] * (1.f + hsc[c + e]));
          *(bf16x8*)(hq + c) = v;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) hq[c] = from_f32<T>(y[c] * (1.f + hsc[c]));
      }
    }
  }
  if (a.stats) {   // uniform (kernel argument)
    // (mean, M2) of the thread's 16 columns, merged with the other 16-column groups of the
    // slot (adjacent lanes of the row); rows past the end still join the shuffles
    static_assert(kStatCols % 16 == 0 && 64 % kStatCols == 0, "slot groups");
    float mean = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) mean += y[c];
    mean *= (1.f / 16.f);
    float m2 = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) m2 += (y[c] - mean) * (y[c] - mean);
#pragma unroll
    for (int off = 1; off < kStatCols / 16; off <<= 1) {
      const float mb = __shfl_xor(mean, off, 64), qb = __shfl_xor(m2, off, 64);
      const float d = mb - mean;   // equal counts: merged mean is the average
      m2 += qb + d * d * (float)(8 * off);
      mean = 0.5f * (mean + mb);
    }
    if (rok && (g % (kStatCols / 16)) == 0)
      a.stats[(long)hr * a.stats_ld + (n0 + g * 16) / kStatCols] = make_float2(mean, m2);
  }
}

hipError_t inproj_launch(const InProjArgs& in, int elem, hipStream_t s) {
  const int rows = in.B * (in.st + in.Ha);
  if (rows == 0) return hipSuccess;
  if (in.da > kInMaxK || in.D % 64 != 0 || !in.zeros || (long)in.D + 4 > kVecPad) return hipErrorInvalidValue;
  InProjArgs a = in;   // absent optional vectors read zeros
  if (!a.tb) a.tb = a.zeros;
  if (!a.hscale) a.hscale = a.zeros;
  if (!a.state_tok) { a.state_tok = a.zeros; a.st = 0; }
  const dim3 grid(a.D / 64, (rows + 63) / 64);
  if (elem == ET_BF16) hipLaunchKernelGGL(k_inproj<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_inproj<float>, grid, dim3(256), 0, s, a);
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
template <typename T>
__global__ void k_rows_from_f32(T* dst, long dld, const float* src, long sld, int rows, int cols, float add) {
  const long n = (long)rows * cols;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const long r = i / cols, c = i % cols;
    dst[r * dld + c] = from_f32<T>(src[r * sld + c] + add);
  }
}
__global__ void k_xcc_probe(uint32_t* out, int n) {
  if (threadIdx.x == 0 && (int)blockIdx.x < n) out[blockIdx.x] = hw_xcc_id();
}
hipError_t xcc_probe(uint32_t* out, int n, hipStream_t s) {
  if (n < 1 || n > 65536) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_xcc_probe, dim3(n), dim3(64), 0, s, out, n);
  return hipGetLastError();
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
hipError_t rows_from_f32(void* dst, long dld, const float* src, long sld, int rows, int cols, float add, int elem,
                         hipStream_t s) {
  const long n = (long)rows * cols;
  if (n <= 0) return hipSuccess;
  if (elem == ET_BF16)
    hipLaunchKernelGGL(k_rows_from_f32<bf16>, dim3(grid_for(n)), dim3(256), 0, s, (bf16*)dst, dld, src, sld, rows, cols, add);
  else
    hipLaunchKernelGGL(k_rows_from_f32<float>, dim3(grid_for(n)), dim3(256), 0, s, (float*)dst, dld, src, sld, rows, cols, add);
  return hipGetLastError();
}

// The step after the path: a model-space chunk [B][H][da] back to robot units
// [B][hr][dr] with per-dimension (q01, q99), and cut to the first hr steps and dr dims.
// kind 0 (pi0.5 Design, "Embodiment adapters": openpi's quantile normalization inverted,
// epsilon included): (x + 1) / 2 * (q99 - q01 + 1e-6) + q01. kind 1 (GR00T N1.7, "Policy
// contract"): (clip(x, -1, 1) + 1) / 2 * (q99 - q01) + q01. One thread per output element.
__global__ void k_unnormalize(const float* __restrict__ x, float* __restrict__ out, const float* __restrict__ q01,
                              const float* __restrict__ q99, int B, int H, int da, int hr, int dr, int kind) {
  const long n = (long)B * hr * dr;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int j = (int)(i % dr);
    const long bt = i / dr;
    const int t = (int)(bt % hr), b = (int)(bt / hr);
    float v = x[((long)b * H + t) * da + j];
    const float lo = q01[j], hi = q99[j];
    if (kind == 0) {
      out[i] = (v + 1.f) * 0.5f * (hi - lo + 1e-6f) + lo;
    } else {
      v = fminf(fmaxf(v, -1.f), 1.f);
      out[i] = (v + 1.f) * 0.5f * (hi - lo) + lo;
    }
  }
}

hipError_t unnormalize_launch(const float* x, float* out, const float* q01, const float* q99, int B, int H, int da,
                              int hr, int dr, int kind, hipStream_t s) {
  const long n = (long)B * hr * dr;
  if (n <= 0) return hipSuccess;
  const int grid = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_unnormalize, dim3(grid), dim3(256), 0, s, x, out, q01, q99, B, H, da, hr, dr, kind);
  return hipGetLastError();
}
// FP8 weights: each row of src [N x K] (bf16) as E4M3 codes times 2^e_row, e_row the smallest
// exponent with max |row| <= 448 2^e (max = f 2^x, f in [0.5, 1): e = x - 9 + [f > 0.875]).
// One workgroup per row. Codes come from the hardware conversion (round to nearest even;
// |x 2^-e| <= 448 cannot overflow); deq = code 2^e in bf16, exact (a code has at most four
// significant bits).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__global__ void __launch_bounds__(256) k_quant_fp8(const bf16* __restrict__ src, long ld, int K, uint8_t* __restrict__ codes,
                                                   float* __restrict__ scale, bf16* __restrict__ deq) {
  __shared__ float red[256];
  const long r = blockIdx.x;
  const bf16* row = src + r * ld;
  float m = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) m = fmaxf(m, fabsf((float)row[k]));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float amax = red[0];
  int x = 0;
  const float f = frexpf(amax, &x);
  const int e = amax > 0.f ? x - 9 + (f > 0.875f ? 1 : 0) : 0;
  const float sc = ldexpf(1.f, e);
  if (threadIdx.x == 0) scale[r] = sc;
  for (int k = 2 * (int)threadIdx.x; k < K; k += 512) {   // K even: pairs
    const float q0 = ldexpf((float)row[k], -e), q1 = ldexpf((float)row[k + 1], -e);
    const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);   // codes in bits [15:0]
    *(uint16_t*)(codes + r * K + k) = (uint16_t)(w & 0xFFFFu);
    *(bf16x2*)(deq + r * K + k) = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, false);
  }
}

// FP8 weights fragment-major: fragment (nb, kp) = rows 16 nb .. 16 nb + 15 x k 64 kp .. 64 kp
// + 63, 1 KB; lane l holds row 16 nb + l % 16: bytes 0-7 the codes of k = 64 kp + 8 (l / 16)
// + 0..7, bytes 8-15 those of k + 32 (two 32-wide MFMA k-chunks). rows: source row of each
// output row (null = identity). Rows past N are zeros.
__global__ void k_swizzle_fp8(uint8_t* __restrict__ dst, const uint8_t* __restrict__ codes, const int* __restrict__ rows,
                              int N, int K) {
  const int KP = K / 64;
  const long nfrag = (long)((N + 15) / 16) * KP;
  for (long c = blockIdx.x * (long)blockDim.x + threadIdx.x; c < nfrag * 64; c += (long)gridDim.x * blockDim.x) {
    const long fidx = c / 64;
    const int l = (int)(c % 64);
    const int nb = (int)(fidx / KP), kp = (int)(fidx % KP);
    const int n = nb * 16 + (l % 16);
    const int k = kp * 64 + (l / 16) * 8;
    uint2 lo = make_uint2(0u, 0u), hi = lo;
    if (n < N) {
      const int sr = rows ? rows[n] : n;
      lo = *(const uint2*)(codes + (long)sr * K + k);
      hi = *(const uint2*)(codes + (long)sr * K + k + 32);
    }
    *(uint4*)(dst + c * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

__global__ void k_gather_f32(float* __restrict__ dst, const float* __restrict__ src, const int* __restrict__ rows, int N, int Npad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < Npad) dst[i] = i < N ? src[rows ? rows[i] : i] : 0.f;
}

hipError_t quantize_fp8_rows(const void* src, long ld, int N, int K, uint8_t* codes, float* scale, void* deq, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (K % 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quant_fp8, dim3(N), dim3(256), 0, s, (const bf16*)src, ld, K, codes, scale, (bf16*)deq);
  return hipGetLastError();
}

size_t swizzled_fp8_bytes(int N, int K) { return (size_t)((N + 15) / 16) * 16 * K; }

hipError_t swizzle_fp8(void* dst, const uint8_t* codes, const int* rows, int N, int K, hipStream_t s) {
  if (K % 64) return hipErrorInvalidValue;
  const long n = (long)((N + 15) / 16) * (K / 64) * 64;
  hipLaunchKernelGGL(k_swizzle_fp8, dim3(grid_for(n)), dim3(256), 0, s, (uint8_t*)dst, codes, rows, N, K);
  return hipGetLastError();
}

hipError_t gather_f32(float* dst, const float* src, const int* rows, int N, int Npad, hipStream_t s) {
  if (Npad <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_f32, dim3((Npad + 255) / 256), dim3(256), 0, s, dst, src, rows, N, Npad);
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
// pool[b*pool_bs + d*cap + vt_slot(j)] = src[(b*P + j)*dh + d]
template <typename T>
__global__ void k_prefix_vt(T* pool, long pool_bs, int cap, const T* src, int B, int P, int dh) {
  const long n = (long)B * P * dh;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int j = (int)(i % P);
    const long r = i / P;
    const int d = (int)(r % dh), b = (int)(r / dh);
    pool[(long)b * pool_bs + (long)d * cap + vt_slot<T>(j)] = src[((long)b * P + j) * dh + d];
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
