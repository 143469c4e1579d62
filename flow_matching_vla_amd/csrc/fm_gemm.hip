// MFMA GEMM for the action expert: C = A W^T with fused prologue (RMS/Layer norm +
// (1 + scale) / shift modulation applied while staging A) and fused epilogues (bias +
// activation store, GELU(gate) * up, Q/K RoPE with K/V append, gated residual with row
// statistics, velocity projection + Euler update). gfx950, bf16 or fp32 operands, fp32
// accumulation. Weights are kept in a fragment-major layout so that every 16-byte lane
// load of a weight tile is part of one contiguous 1 KB run.
#include "fm_common.h"
#include "fm_kernels.h"

namespace fm {

// ---------------------------------------------------------------------------------------
// Fragment-major weight layout. Fragment (nb, kc) covers rows [16 nb, 16 nb + 16) and
// k in [KC kc, KC kc + KC); lane l of it holds row 16 nb + l % 16, k = KC kc + (l/16) VEC
// .. + VEC - 1. Fragments are ordered nb-major: ((nb * KB + kc) * 64 + l) * VEC elements.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ void k_swizzle(T* __restrict__ dst, const T* __restrict__ src, const int* __restrict__ rows,
                          int N, int K, long ld) {
  constexpr int VEC = Mma<T>::VEC, KC = Mma<T>::KC;
  const int KB = K / KC;
  const long nfrag = (long)((N + 15) / 16) * KB;
  for (long c = blockIdx.x * (long)blockDim.x + threadIdx.x; c < nfrag * 64; c += (long)gridDim.x * blockDim.x) {
    const long f = c / 64;
    const int l = (int)(c % 64);
    const int nb = (int)(f / KB), kc = (int)(f % KB);
    const int n = nb * 16 + (l % 16);
    const int k = kc * KC + (l / 16) * VEC;
    V16 v = {{0, 0, 0, 0}};
    if (n < N) {
      const int sr = rows ? rows[n] : n;
      if (sr >= 0) v = *(const V16*)(src + (long)sr * ld + k);
    }
    *(V16*)(dst + c * VEC) = v;
  }
}

size_t swizzled_bytes(int N, int K, int elem) {
  return (size_t)((N + 15) / 16) * 16 * K * (elem == ET_BF16 ? 2 : 4);
}

hipError_t swizzle_weight(void* dst, const void* src, const int* rows, int N, int K, long ld, int elem,
                          hipStream_t s) {
  const long n16 = (long)((N + 15) / 16) * 16 * K / (elem == ET_BF16 ? 8 : 4);
  const int grid = (int)((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096);
  if (elem == ET_BF16)
    hipLaunchKernelGGL(k_swizzle<bf16>, dim3(grid), dim3(256), 0, s, (bf16*)dst, (const bf16*)src, rows, N, K, ld);
  else
    hipLaunchKernelGGL(k_swizzle<float>, dim3(grid), dim3(256), 0, s, (float*)dst, (const float*)src, rows, N, K, ld);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Row statistics: (mean, M2) over a run of columns, merged pairwise (Chan et al.).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void stat_merge(float& mean, float& m2, float n, float mean_b, float m2_b, float n_b) {
  const float tot = n + n_b;
  const float d = mean_b - mean;
  mean += d * (n_b / tot);
  m2 += m2_b + d * d * (n * n_b / tot);
}

// ---------------------------------------------------------------------------------------
// Epilogue over a BM x BN fp32 tile held in LDS (row stride LDC). Items are 4-column
// runs; the 16 consecutive lanes that share a row cover 64 columns = one statistic slot.
// ---------------------------------------------------------------------------------------
template <typename T, int BM, int BN, int NT, int EPI>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& a, const float* C, int ldc, int m0, int n0) {
  constexpr int C4 = BN / 4;
  const int tid = threadIdx.x;
  for (int it = tid; it < BM * C4; it += NT) {
    const int r = it / C4, c4 = it % C4;
    const int m = m0 + r;
    const int n = n0 + c4 * 4;
    const bool mok = m < a.M;
    float v[4];
    {
      const f32x4 cv = *(const f32x4*)(C + r * ldc + c4 * 4);
      v[0] = cv[0]; v[1] = cv[1]; v[2] = cv[2]; v[3] = cv[3];
    }
    if constexpr (EPI == EPI_STORE) {
      if (mok) {
        for (int j = 0; j < 4; ++j) {
          if (n + j >= a.N) break;
          float y = v[j] + (a.bias ? a.bias[n + j] : 0.f);
          if (a.act == ACT_SILU) y = silu(y);
          else if (a.act == ACT_GELU) y = gelu_tanh(y);
          if (a.out_f32) ((float*)a.out)[(long)m * a.ldo + n + j] = y;
          else ((T*)a.out)[(long)m * a.ldo + n + j] = from_f32<T>(y);
        }
      }
    } else if constexpr (EPI == EPI_GELU_MUL) {
      // columns interleave (gate_f, up_f) pairs: output f = n / 2
      if (mok) {
        for (int j = 0; j < 4; j += 2) {
          if (n + j + 1 >= a.N + 1) break;
          const float y = gelu_tanh(v[j]) * v[j + 1];
          ((T*)a.out)[(long)m * a.ldo + (n + j) / 2] = from_f32<T>(y);
        }
      }
    } else if constexpr (EPI == EPI_QKV) {
      if (mok) {
        const int b = m / a.tq, i = m % a.tq;
        if (n < a.q_cols + a.kv_cols && a.rope) {
          // pairs (2j, 2j + 1) of the interleaved head layout rotate together
          const int c = n < a.q_cols ? n : n - a.q_cols;
          const int dh = 2 * a.half_dh;
          for (int j = 0; j < 4; j += 2) {
            const int jj = ((c + j) % dh) / 2;
            const float2 cs = a.rope_cs[(long)i * a.half_dh + jj];
            const float x0 = v[j], x1 = v[j + 1];
            v[j] = x0 * cs.x - x1 * cs.y;
            v[j + 1] = x1 * cs.x + x0 * cs.y;
          }
        }
        for (int j = 0; j < 4; ++j) {
          const int nn = n + j;
          if (nn >= a.N) break;
          if (nn < a.q_cols) {
            ((T*)a.out)[(long)m * a.ldo + nn] = from_f32<T>(v[j]);
          } else if (nn < a.q_cols + a.kv_cols) {
            const int c = nn - a.q_cols;
            ((T*)a.kdst)[(long)b * a.k_bs + (long)(a.kv_off + i) * a.k_rs + c] = from_f32<T>(v[j]);
          } else {
            const int c = nn - a.q_cols - a.kv_cols;
            ((T*)a.vdst)[(long)b * a.v_bs + (long)c * a.v_ds + a.kv_off + i] = from_f32<T>(v[j]);
          }
        }
      }
    } else if constexpr (EPI == EPI_VT) {
      if (mok) {
        const int b = m / a.vt_group, s = m % a.vt_group;
        for (int j = 0; j < 4; ++j) {
          if (n + j >= a.N) break;
          ((T*)a.out)[(long)b * a.vt_bs + (long)(n + j) * a.vt_ds + s] = from_f32<T>(v[j]);
        }
      }
    } else if constexpr (EPI == EPI_RESID) {
      // h += gate * acc, then (mean, M2) of the updated 64-column slot for the next norm.
      // N is a multiple of BN here, so every item is in range column-wise.
      float hv[4] = {0.f, 0.f, 0.f, 0.f};
      if (mok) {
        float* hp = a.h + (long)m * a.ldh_out + n;
        const f32x4 ho = *(const f32x4*)hp;
        for (int j = 0; j < 4; ++j) hv[j] = ho[j] + (a.gate ? a.gate[n + j] : 1.f) * v[j];
        f32x4 hn; hn[0] = hv[0]; hn[1] = hv[1]; hn[2] = hv[2]; hn[3] = hv[3];
        *(f32x4*)hp = hn;
      }
      float mean = 0.25f * (hv[0] + hv[1] + hv[2] + hv[3]);
      float m2 = 0.f;
      for (int j = 0; j < 4; ++j) m2 += (hv[j] - mean) * (hv[j] - mean);
      float cnt = 4.f;
      for (int off = 1; off < 16; off <<= 1) {
        const float mb = __shfl_xor(mean, off, 64);
        const float qb = __shfl_xor(m2, off, 64);
        stat_merge(mean, m2, cnt, mb, qb, cnt);
        cnt *= 2.f;
      }
      if (mok && (c4 % 16) == 0) {
        const int part = n / kStatCols;
        a.stats_out[(long)part * a.stats_out_ld + m] = make_float2(mean, m2);
      }
    } else if constexpr (EPI == EPI_EULER) {
      if (mok) {
        for (int j = 0; j < 4; ++j) {
          if (n + j >= a.N) break;
          const float vel = v[j] + (a.bias ? a.bias[n + j] : 0.f);
          const long idx = (long)m * a.ldo + n + j;
          if (a.vout) a.vout[idx] = vel;
          if (a.x) a.x[idx] += a.dt * vel;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// The GEMM kernel. Workgroup = WM x WN waves; tile BM x BN; k-tile BK; two LDS stages in
// fragment-major order (conflict-free 16-byte reads); optional split-K over workgroups with
// the last-arriving workgroup of a tile summing the partials in split order.
// ---------------------------------------------------------------------------------------
template <typename T, int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ void __launch_bounds__(WM* WN * 64) k_gemm(GemmArgs a) {
  using MT = Mma<T>;
  typedef typename MT::frag frag;
  constexpr int NT = WM * WN * 64;
  constexpr int VEC = MT::VEC, KC = MT::KC;
  constexpr int KCH = BK / KC;                // k-chunks per k-tile
  constexpr int SEG = KC / VEC;               // 16-byte segments per chunk row (4)
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_CH = BM * BK / VEC, B_CH = BN * BK / VEC;
  constexpr int A_PT = (A_CH + NT - 1) / NT, B_PT = (B_CH + NT - 1) / NT;
  constexpr int STAGE_V16 = A_CH + B_CH;
  constexpr int LDC = BN + 4;
  constexpr int SMEM_MAIN = 2 * STAGE_V16 * 16;
  constexpr int SMEM_EPI = BM * LDC * 4;
  constexpr int SMEM = SMEM_MAIN > SMEM_EPI ? SMEM_MAIN : SMEM_EPI;
  static_assert(BK % KC == 0 && BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile");
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ float s_mean[BM], s_rinv[BM];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int ntn = (a.N + BN - 1) / BN, ntm = (a.M + BM - 1) / BM;
  const int tiles = ntn * ntm;
  const int bid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int split = bid / tiles, t = bid % tiles;
  const int tn = t % ntn, tm = t / ntn;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KB = a.K / KC;                    // k-chunks in the full K (weights layout)
  const int kbeg = split * a.k_split;
  const int kend = min(a.K, kbeg + a.k_split);
  const int nkt = (kend - kbeg + BK - 1) / BK;
  const bool normed = a.norm != NORM_NONE;

  if (normed) {
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      float mean = 0.f, rinv = 0.f;
      if (m < a.M) {
        const int hr = (m / a.row_group) * a.row_gstride + a.row_off + m % a.row_group;
        float mu = 0.f, m2 = 0.f, cnt = 0.f;
        for (int p = 0; p < a.nparts; ++p) {
          const float2 st = a.stats[(long)p * a.stats_ld + hr];
          if (p == 0) { mu = st.x; m2 = st.y; cnt = (float)kStatCols; }
          else { stat_merge(mu, m2, cnt, st.x, st.y, (float)kStatCols); cnt += (float)kStatCols; }
        }
        if (a.norm == NORM_RMS) {
          const float ms = (m2 + cnt * mu * mu) / cnt;
          rinv = rsqrtf(ms + a.eps);
          mean = 0.f;
        } else {
          rinv = rsqrtf(m2 / cnt + a.eps);
          mean = mu;
        }
      }
      s_mean[r] = mean;
      s_rinv[r] = rinv;
    }
    __syncthreads();
  }

  V16 ra[A_PT][2];
  V16 rb[B_PT];
  V16* lds = (V16*)smem;

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int p = 0; p < A_PT; ++p) {
      const int c = tid + p * NT;
      ra[p][0] = V16{{0, 0, 0, 0}};
      ra[p][1] = V16{{0, 0, 0, 0}};
      if (c < A_CH) {
        const int r = c / (BK / VEC), ks = c % (BK / VEC);
        const int m = m0 + r, k = k0 + ks * VEC;
        if (m < a.M && k < kend) {
          if (!normed) {
            ra[p][0] = *(const V16*)((const T*)a.A + (long)m * a.lda + k);
          } else {
            const int hr = (m / a.row_group) * a.row_gstride + a.row_off + m % a.row_group;
            const float* hp = a.H + (long)hr * a.ldh + k;
            ra[p][0] = *(const V16*)hp;
            if (VEC == 8) ra[p][1] = *(const V16*)(hp + 4);
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < B_PT; ++p) {
      const int c = tid + p * NT;
      rb[p] = V16{{0, 0, 0, 0}};
      if (c < B_CH) {
        const int f = c / 64, slot = c % 64;
        const int nbl = f / KCH, kcl = f % KCH;
        const int nb = n0 / 16 + nbl, kc = k0 / KC + kcl;
        if (nb * 16 < a.N && kc * KC < kend)
          rb[p] = *((const V16*)a.W + ((long)nb * KB + kc) * 64 + slot);
      }
    }
  };

  auto store_tile = [&](int stage, int k0) {
    V16* As = lds + stage * STAGE_V16;
    V16* Bs = As + A_CH;
#pragma unroll
    for (int p = 0; p < A_PT; ++p) {
      const int c = tid + p * NT;
      if (c < A_CH) {
        const int r = c / (BK / VEC), ks = c % (BK / VEC);
        V16 val = ra[p][0];
        if (normed) {
          const int m = m0 + r, k = k0 + ks * VEC;
          float f[8];
          if (m < a.M && k < kend) {
            unpack<float>(ra[p][0], f);
            if (VEC == 8) unpack<float>(ra[p][1], f + 4);
            const float mu = s_mean[r], ri = s_rinv[r];
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
              float u = (f[j] - mu) * ri;
              if (a.mscale) u = u * (1.f + a.mscale[k + j]) + a.mshift[k + j];
              f[j] = u;
            }
          } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) f[j] = 0.f;
          }
          val = pack<T>(f);
        }
        const int frag_i = (r / 16) * KCH + ks / SEG;
        const int slot = (r % 16) + 16 * (ks % SEG);
        As[frag_i * 64 + slot] = val;
      }
    }
#pragma unroll
    for (int p = 0; p < B_PT; ++p) {
      const int c = tid + p * NT;
      if (c < B_CH) Bs[c] = rb[p];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nkt > 0) {
    load_tile(kbeg);
    store_tile(0, kbeg);
    __syncthreads();
    for (int it = 0; it < nkt; ++it) {
      const int cur = it & 1;
      const int knext = kbeg + (it + 1) * BK;
      if (it + 1 < nkt) load_tile(knext);
      const V16* As = lds + cur * STAGE_V16;
      const V16* Bs = As + A_CH;
#pragma unroll
      for (int kc = 0; kc < KCH; ++kc) {
        frag af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const V16 v = As[((wm * FM + i) * KCH + kc) * 64 + lane];
          af[i] = __builtin_bit_cast(frag, v);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const V16 v = Bs[((wn * FN + j) * KCH + kc) * 64 + lane];
          bfr[j] = __builtin_bit_cast(frag, v);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = MT::mma(af[i], bfr[j], acc[i][j]);
      }
      if (it + 1 < nkt) store_tile(cur ^ 1, knext);
      __syncthreads();
    }
  }

  // accumulators -> LDS tile (row-major, fp32)
  float* C = (float*)smem;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = wm * TM + i * 16 + 4 * (lane / 16) + e;
        const int c = wn * TN + j * 16 + (lane % 16);
        C[r * LDC + c] = acc[i][j][e];
      }
  __syncthreads();

  if (a.splits > 1) {
    float* wst = a.ws + (long)t * a.splits * BM * BN;
    for (int it = tid; it < BM * BN / 4; it += NT) {
      const int r = it / (BN / 4), c4 = it % (BN / 4);
      *(f32x4*)(wst + (long)split * BM * BN + r * BN + c4 * 4) = *(const f32x4*)(C + r * LDC + c4 * 4);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(a.counters + t, 1u);
      s_last = (prev == (unsigned)a.splits - 1u);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int it = tid; it < BM * BN / 4; it += NT) {
      const int r = it / (BN / 4), c4 = it % (BN / 4);
      f32x4 s = *(const f32x4*)(wst + r * BN + c4 * 4);
      for (int sp = 1; sp < a.splits; ++sp) s += *(const f32x4*)(wst + (long)sp * BM * BN + r * BN + c4 * 4);
      *(f32x4*)(C + r * LDC + c4 * 4) = s;
    }
    if (tid == 0) a.counters[t] = 0u;
    __syncthreads();
  }
  epilogue_tile<T, BM, BN, NT, EPI>(a, C, LDC, m0, n0);
}

// ---------------------------------------------------------------------------------------
// Host side: planning and dispatch.
// ---------------------------------------------------------------------------------------
struct CfgShape { int bm, bn, bk; };
static CfgShape cfg_shape(int cfg, int elem) {
  const int bk = elem == ET_BF16 ? 64 : 32;
  switch (cfg) {
    case GEMM_128x128: return {128, 128, bk};
    case GEMM_32x64: return {32, 64, bk};
    default: return {64, 64, bk};
  }
}

int gemm_num_tiles(const GemmArgs& a) {
  const CfgShape c = cfg_shape(a.cfg, a.epi == EPI_RESID ? ET_BF16 : ET_BF16);
  return ((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn);
}

void gemm_plan(GemmArgs& a, int elem, int num_cus) {
  // Large M: 128 x 128 tiles. Small M: 64-row (or 32-row) tiles with split-K until the
  // launch covers the chip about twice.
  if (elem == ET_BF16 && a.M >= 256 && a.N >= 512) a.cfg = GEMM_128x128;
  else if (a.M <= 32) a.cfg = GEMM_32x64;
  else a.cfg = GEMM_64x64;
  const CfgShape c = cfg_shape(a.cfg, elem);
  const int tiles = ((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn);
  const int nk = (a.K + c.bk - 1) / c.bk;
  int splits = 1;
  const int target = 2 * num_cus;
  if (tiles < target) {
    splits = (target + tiles - 1) / tiles;
    const int max_splits = nk / 2 > 0 ? nk / 2 : 1;   // at least two k-tiles per split
    if (splits > max_splits) splits = max_splits;
    if (splits > 32) splits = 32;
  }
  int kt_per = (nk + splits - 1) / splits;
  splits = (nk + kt_per - 1) / kt_per;
  a.splits = splits;
  a.k_split = kt_per * c.bk;
}

size_t gemm_ws_bytes(const GemmArgs& a) {
  if (a.splits <= 1) return 0;
  const CfgShape c = cfg_shape(a.cfg, ET_BF16);
  const int tiles = ((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn);
  return (size_t)tiles * a.splits * c.bm * c.bn * sizeof(float);
}

template <typename T, int BM, int BN, int BK, int WM, int WN>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const dim3 grid(tiles * a.splits), block(WM * WN * 64);
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, EPI_STORE>), grid, block, 0, s, a); break;
    case EPI_GELU_MUL: hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, EPI_GELU_MUL>), grid, block, 0, s, a); break;
    case EPI_QKV: hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, EPI_QKV>), grid, block, 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, EPI_RESID>), grid, block, 0, s, a); break;
    case EPI_EULER: hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, EPI_EULER>), grid, block, 0, s, a); break;
    case EPI_VT: hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, EPI_VT>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t gemm_launch(const GemmArgs& a, int elem, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (elem == ET_BF16) {
    switch (a.cfg) {
      case GEMM_128x128: return launch_cfg<bf16, 128, 128, 64, 2, 2>(a, s);
      case GEMM_32x64: return launch_cfg<bf16, 32, 64, 64, 1, 4>(a, s);
      default: return launch_cfg<bf16, 64, 64, 64, 2, 2>(a, s);
    }
  }
  switch (a.cfg) {
    case GEMM_32x64: return launch_cfg<float, 32, 64, 32, 1, 4>(a, s);
    default: return launch_cfg<float, 64, 64, 32, 2, 2>(a, s);
  }
}

}  // namespace fm
