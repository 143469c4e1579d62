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
    V16 v = vzero();
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

__device__ __forceinline__ int a_row(const GemmArgs& a, int m) {
  return (m / a.row_group) * a.row_gstride + a.row_off + m % a.row_group;
}

// Per-row (mu, rinv) of the BM rows starting at m0, from the producer's per-slot partial
// statistics stats[row][slot] (slots of kStatCols columns). TPR = NT / BM threads share a
// row; each reads PPT 16-byte slot pairs at a stride of TPR pairs and the partial sums are
// merged across the row's lanes. Split in two so that the slot loads are issued together
// with the operand loads and merged after them. Loads past the row's slots read the next
// row (or the buffer's tail padding) and are masked out.
template <int BM, int NT>
struct RowStats {
  static constexpr int TPR = NT / BM;
  static constexpr int PPT = (kMaxStatSlots / 2 + TPR - 1) / TPR;
  static_assert(TPR >= 1 && (TPR & (TPR - 1)) == 0 && TPR <= 64, "threads per row");
  f32x4 v[PPT];
  __device__ __forceinline__ void load(const GemmArgs& a, int m0) {
    const int tid = threadIdx.x;
    const int r = tid / TPR, q = tid % TPR;
    const float2* rp = a.stats + (long)a_row(a, min(m0 + r, a.M - 1)) * a.stats_ld + 2 * q;
#pragma unroll
    for (int u = 0; u < PPT; ++u) v[u] = *(const f32x4*)(rp + 2 * u * TPR);
  }
  __device__ __forceinline__ void merge(const GemmArgs& a, int m0, float* s_mean, float* s_rinv) {
    // every slot covers kStatCols columns: mean = average of slot means, and
    // M2 = sum of slot M2 + kStatCols * sum (slot mean - mean)^2
    const int tid = threadIdx.x;
    const int r = tid / TPR, q = tid % TPR;
    float sm = 0.f;
#pragma unroll
    for (int u = 0; u < PPT; ++u) sm += (2 * (q + u * TPR) < a.nparts) ? v[u][0] + v[u][2] : 0.f;
    sm = group_sum<TPR>(sm);
    const float np = (float)a.nparts;
    const float mu = sm / np;
    float m2 = 0.f;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const float d0 = v[u][0] - mu, d1 = v[u][2] - mu;
      m2 += (2 * (q + u * TPR) < a.nparts) ? v[u][1] + v[u][3] + (float)kStatCols * (d0 * d0 + d1 * d1) : 0.f;
    }
    m2 = group_sum<TPR>(m2);
    if (q == 0 && r < BM) {
      const float cnt = np * (float)kStatCols;
      const bool ok = m0 + r < a.M;
      float mean = 0.f, rinv;
      if (a.norm == NORM_RMS) {
        rinv = rsqrtf((m2 + cnt * mu * mu) / cnt + a.eps);
      } else {
        rinv = rsqrtf(m2 / cnt + a.eps);
        mean = mu;
      }
      s_mean[r] = ok ? mean : 0.f;
      s_rinv[r] = ok ? rinv : 0.f;
    }
  }
};

// Device-scope (sc1) 16-byte accesses for partial tiles exchanged between workgroups of one
// kernel: written through to, and read back from, the device-coherent level without a
// write-back or invalidation of the whole L2. Offsets are in bytes from the workspace base.
constexpr int kCpolSc1 = 16;             // cache-policy operand: sc1
constexpr uint32_t kOob = 0x80000000u;   // byte offset past every buffer extent (all < 2^31)
__device__ __forceinline__ void st_dev(const Rsrc& r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(V16, v), r, off, 0, kCpolSc1);
}
__device__ __forceinline__ f32x4 ld_dev(const Rsrc& r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1));
}
// XCD-local exchange (all parties on one XCD, which has one L2): plain stores (the vector
// L1 writes through to L2), an arrival counter updated by atomics that execute in L2, and
// device-scope (sc1) loads, which miss the reader's L1 (an L1 invalidate does not serve: the
// workgroup-scope form drops nothing, and the agent-scope form also drops the L2's lines).
__device__ __forceinline__ void st_l2(const Rsrc& r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(V16, v), r, off, 0, 0);
}
__device__ __forceinline__ f32x4 ld_l2(const Rsrc& r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1));
}
__device__ __forceinline__ uint32_t l2_fetch_add(unsigned* p, uint32_t v) {
  uint32_t old;
  asm volatile("global_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(old) : "v"(p), "v"(v) : "memory");
  return old;
}
__device__ __forceinline__ void l2_put(unsigned* p, uint32_t v) {
  __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------------------
// Epilogue over a BM x BN fp32 tile held in LDS (row stride ldc). Items are 4-column runs;
// four consecutive lanes of a row cover one 16-column statistic slot. Every global input
// (bias, modulation vectors, residual, x, RoPE table) is loaded for all of the thread's
// items before any is used.
// ---------------------------------------------------------------------------------------
// four / two consecutive outputs as one store (address aligned to its size)
template <typename T> __device__ __forceinline__ void store4(T* o, const float* y);
template <> __device__ __forceinline__ void store4<float>(float* o, const float* y) { *(f32x4*)o = f32x4{y[0], y[1], y[2], y[3]}; }
template <> __device__ __forceinline__ void store4<bf16>(bf16* o, const float* y) {
  *(bf16x4*)o = bf16x4{(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
}
template <typename T> __device__ __forceinline__ void store2(T* o, float y0, float y1);
template <> __device__ __forceinline__ void store2<float>(float* o, float y0, float y1) { *(float2*)o = make_float2(y0, y1); }
template <> __device__ __forceinline__ void store2<bf16>(bf16* o, float y0, float y1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  *(bf16x2*)o = bf16x2{(bf16)y0, (bf16)y1};
}

// Wait until at most n vector-memory operations of this wave are in flight. Issued through
// the compiler's own intrinsic, so its wait tracking knows every older load has landed.
#define FM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

template <typename T, int BM, int BN, int NT, int EPI>
struct Epilogue {
  static constexpr int C4 = BN / 4;
  static constexpr int TOT = BM * C4;
  static constexpr int ITEMS = (TOT + NT - 1) / NT;
  static_assert(TOT % 64 == 0 && C4 % 4 == 0, "epilogue items");
  static_assert(EPI != EPI_RESID || BN % kStatCols == 0, "residual tiles cover whole statistic slots");
  static_assert(NT % C4 == 0, "every item of a thread is the same 4-column run");
  // per-column inputs of the thread's column run (c, d, bias, gate, next scale) and the
  // per-item row inputs (residual h, state x, RoPE cos/sin)
  f32x4 pc, pd, pb, pg, ps;
  f32x4 pr[ITEMS];

  // Loads use clamped indices and are unconditional (a divergent conditional load costs a
  // full memory round trip of its own); values outside the tile are never used. Per-column
  // vectors are padded to a multiple of four floats by their owners, and the launcher has
  // replaced every absent one by a zeros (gate: ones) buffer.
  static __device__ __forceinline__ f32x4 vec4(const float* p, long i) { return *(const f32x4*)(p + i); }

  __device__ __forceinline__ void prefetch_cols(const GemmArgs& a, int n0) {
    const int n = min(n0 + (int)(threadIdx.x % C4) * 4, ((a.N - 1) / 4) * 4);
    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
    pc = vec4(a.cvec, n);
    pd = vec4(a.dvec, n);
    pb = z; pg = z; ps = z;
    if constexpr (EPI == EPI_STORE || EPI == EPI_EULER) pb = vec4(a.bias, n);
    if constexpr (EPI == EPI_RESID) { pg = vec4(a.gate, n); ps = vec4(a.hscale, n); }
  }
  __device__ __forceinline__ void prefetch_rows(const GemmArgs& a, int m0, int n0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) {
      const int it = min(tid + q * NT, TOT - 1);
      const int r = it / C4, c4 = it % C4;
      const int mc = min(m0 + r, a.M - 1), n = min(n0 + c4 * 4, ((a.N - 1) / 4) * 4);
      pr[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (EPI == EPI_EULER) pr[q] = vec4(a.x, (long)mc * a.ldo + n);
      if constexpr (EPI == EPI_RESID) pr[q] = vec4(a.h, (long)mc * a.ldh_out + n);
      if constexpr (EPI == EPI_QKV) {
        const int nr = max(min(n, a.q_cols + a.kv_cols - 4), 0);
        const int c = nr < a.q_cols ? nr : nr - a.q_cols;
        const int jj = (c % max(2 * a.half_dh, 1)) / 2;   // even: pairs jj, jj + 1 are adjacent
        pr[q] = vec4((const float*)a.rope_cs, 2L * ((long)mc * a.half_dh + jj));   // [row][half_dh]
      }
    }
  }
  // the epilogue's global inputs for the thread's items (issued early by the caller)
  __device__ __forceinline__ void prefetch(const GemmArgs& a, int m0, int n0) {
    prefetch_cols(a, n0);
    prefetch_rows(a, m0, n0);
  }
  // Land every prefetched input before the first store. On gfx9 one counter covers loads
  // and stores, so a value loaded before a store can only be waited for together with that
  // store; and the per-item branches keep the compiler from proving that an input has
  // already landed, so without this it waits (stores included) before every item.
  static constexpr bool ROWS = EPI == EPI_RESID || EPI == EPI_QKV || EPI == EPI_EULER;
  static __device__ __forceinline__ void settle() { FM_WAIT_VM(0); }

  // A tile of V columns only, stored transposed ([d][key] planes). Its items walk the rows
  // (lane = row of the 64-row slab), so each store instruction writes 64 keys of one
  // transposed row instead of 64 scattered keys. An item's four columns are then the same
  // for the whole wave, so its norm vectors are scalar loads (waited on the scalar counter:
  // no store of this call is waited for).
  __device__ __forceinline__ void apply_vt(const GemmArgs& a, const float* C, int ldc, int m0, int n0,
                                           const float* s_mean, const float* s_rinv) {
    typedef const __attribute__((address_space(4))) f32x4 CF4;
    const int tid = threadIdx.x;
    const bool consumer = a.norm != NORM_NONE;
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) {
      const int it = tid + q * NT;
      if (it >= TOT) continue;   // uniform per wave
      const int r = it % 64, c4 = it / 64;
      const int m = m0 + r, n = n0 + c4 * 4;
      f32x4 v = *(const f32x4*)(C + r * ldc + c4 * 4);
      if (consumer) {
        const int nu = __builtin_amdgcn_readfirstlane(min(n, ((a.N - 1) / 4) * 4));
        const f32x4 cc = *(CF4*)(a.cvec + nu), dd = *(CF4*)(a.dvec + nu);
        v = s_rinv[r] * (v - s_mean[r] * dd) + cc;
      }
      if (m < a.M && n < a.N) {
        const int b = m / a.tq, i = m % a.tq;
        const int c = n - a.q_cols - a.kv_cols;
        T* o = (T*)a.vdst + (long)b * a.v_bs + vt_slot<T>(a.kv_off + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[(long)(c + j) * a.v_ds] = from_f32<T>(v[j]);
      }
    }
  }

  // y from the fp32 tile C (row stride ldc), then the kind's transform and stores
  __device__ __forceinline__ void apply(const GemmArgs& a, const float* C, int ldc, int m0, int n0,
                                        const float* s_mean, const float* s_rinv) {
  const int tid = threadIdx.x;
  const bool consumer = a.norm != NORM_NONE;
  // A tile of V columns only is stored transposed ([d][key] planes): its items walk the
  // rows (lane = row of a 64-row slab), so that each store instruction writes 64 keys of
  // one transposed row instead of 64 scattered keys.
  if constexpr (EPI == EPI_QKV && BM == 64) {
    if (n0 >= a.q_cols + a.kv_cols) {   // uniform: a tile of V columns only
      apply_vt(a, C, ldc, m0, n0, s_mean, s_rinv);
      return;
    }
  }
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const int it = tid + q * NT;
    if (it >= TOT) continue;   // uniform per wave (TOT is a multiple of 64)
    const int r = it / C4, c4 = it % C4;
    const int m = m0 + r, n = n0 + c4 * 4;
    const bool mok = m < a.M;
    f32x4 v = *(const f32x4*)(C + r * ldc + c4 * 4);
    if (consumer) {
      const float mu = s_mean[r], ri = s_rinv[r];
      v = ri * (v - mu * pd) + pc;   // absent c / d read as zeros
    }
    if constexpr (EPI == EPI_STORE) {
      if (mok) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = v[j] + pb[j];
        if (a.act == ACT_SILU) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = silu(y[j]);
        } else if (a.act == ACT_GELU) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = gelu_tanh(y[j]);
        }
        long base = (long)m * a.ldo + n;
        if (a.col_group) base = (long)(n / a.col_group) * a.col_gstride + (long)m * a.ldo + n % a.col_group;
        if (a.out_f32) {
          float* o = (float*)a.out + base;
          if (n + 3 < a.N && (base & 3) == 0) *(f32x4*)o = f32x4{y[0], y[1], y[2], y[3]};
          else for (int j = 0; j < 4; ++j) if (n + j < a.N) o[j] = y[j];
        } else {
          T* o = (T*)a.out + base;
          if (n + 3 < a.N && (base & 3) == 0) store4<T>(o, y);
          else for (int j = 0; j < 4; ++j) if (n + j < a.N) o[j] = from_f32<T>(y[j]);
        }
      }
    } else if constexpr (EPI == EPI_GELU_MUL) {
      // columns interleave (gate_f, up_f): outputs f = n / 2 and n / 2 + 1
      if (mok && n < a.N) {
        T* o = (T*)a.out + (long)m * a.ldo + n / 2;
        const float g0 = gelu_tanh(v[0]) * v[1], g1 = gelu_tanh(v[2]) * v[3];
        if (n + 2 < a.N && ((((long)m * a.ldo + n / 2) & 1) == 0)) store2<T>(o, g0, g1);
        else {
          o[0] = from_f32<T>(g0);
          if (n + 2 < a.N) o[1] = from_f32<T>(g1);
        }
      }
    } else if constexpr (EPI == EPI_QKV) {
      if (mok) {
        const int b = m / a.tq, i = m % a.tq;
        if (a.rope && n < a.q_cols + a.kv_cols) {
          const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
          v[0] = x0 * pr[q][0] - x1 * pr[q][1];
          v[1] = x1 * pr[q][0] + x0 * pr[q][1];
          v[2] = x2 * pr[q][2] - x3 * pr[q][3];
          v[3] = x3 * pr[q][2] + x2 * pr[q][3];
        }
        const float y4[4] = {v[0], v[1], v[2], v[3]};
        if (n < a.q_cols) {
          store4<T>((T*)a.out + (long)m * a.ldo + n, y4);   // q_cols, ldo multiples of 4
        } else if (n < a.q_cols + a.kv_cols) {
          store4<T>((T*)a.kdst + (long)b * a.k_bs + (long)(a.kv_off + i) * a.k_rs + (n - a.q_cols), y4);
        } else if (n < a.N) {
          const int c = n - a.q_cols - a.kv_cols;
          T* o = (T*)a.vdst + (long)b * a.v_bs + vt_slot<T>(a.kv_off + i);
#pragma unroll
          for (int j = 0; j < 4; ++j) o[(long)(c + j) * a.v_ds] = from_f32<T>(v[j]);
        }
      }
    } else if constexpr (EPI == EPI_VT) {
      if (mok) {
        const int b = m / a.vt_group, sidx = m % a.vt_group;
        for (int j = 0; j < 4; ++j) {
          const int nn = n + j;
          const long col = a.col_group ? (long)(nn / a.col_group) * a.col_gstride + (long)(nn % a.col_group) * a.vt_ds
                                       : (long)nn * a.vt_ds;
          if (nn < a.N) ((T*)a.out)[(long)b * a.vt_bs + col + vt_slot<T>(sidx)] = from_f32<T>(v[j]);
        }
      }
    } else if constexpr (EPI == EPI_RESID) {
      // h += gate * y; hs = T(h (1 + next scale)); (mean, M2) of the kStatCols-column slot
      // (eight consecutive lanes of the row). N is a multiple of kStatCols here.
      f32x4 hv = mok ? pr[q] + pg * v : f32x4{0.f, 0.f, 0.f, 0.f};
      if (mok) {
        *(f32x4*)(a.h + (long)m * a.ldh_out + n) = hv;
        float hsv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) hsv[j] = hv[j] * (1.f + ps[j]);
        store4<T>((T*)a.hs + (long)m * a.ldh_out + n, hsv);   // ldh_out, n multiples of 4
      }
      // the slot's lanes hold four columns each: its mean is the mean of their sums, and
      // M2 the sum of their squared deviations from it (two reductions over the group)
      constexpr int G = kStatCols / 4;
      const float mean = group_sum<G>(hv[0] + hv[1] + hv[2] + hv[3]) * (1.f / kStatCols);
      float m2 = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) m2 += (hv[j] - mean) * (hv[j] - mean);
      m2 = group_sum<G>(m2);
      if (mok && (c4 % (kStatCols / 4)) == 0) a.stats_out[(long)m * a.stats_out_ld + n / kStatCols] = make_float2(mean, m2);
    } else if constexpr (EPI == EPI_EULER) {
      if (mok) {
        for (int j = 0; j < 4; ++j) {
          if (n + j >= a.N) break;
          const float vel = v[j] + pb[j];
          const long idx = (long)m * a.ldo + n + j;
          if (a.vout) a.vout[idx] = vel;
          else a.x[idx] = pr[q][j] + a.dt * vel;
        }
      }
    }
  }
  }
};

// ---------------------------------------------------------------------------------------
// Tiled kernel (M > 64): workgroup = WM x WN waves, tile BM x BN, k-tile BK. Global loads
// of k-tiles run two tiles ahead in registers; two LDS stages in fragment-major order
// (conflict-free 16-byte reads). Optional split-K over workgroups: partial tiles go to the
// workspace with device-scope stores and the last-arriving workgroup of a tile sums them
// in split order (deterministic) and runs the epilogue.
// ---------------------------------------------------------------------------------------
template <typename T, int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ void __launch_bounds__(WM* WN * 64) k_gemm(GemmArgs a) {
  typedef Mma<T> MT;
  typedef typename MT::frag frag;
  constexpr int NT = WM * WN * 64;
  constexpr int VEC = MT::VEC, KC = MT::KC;
  constexpr int KCH = BK / KC, SEG = KC / VEC;
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
  const int KB = a.K / KC;
  const int kbeg = split * a.k_split;
  const int kend = min(a.K, kbeg + a.k_split);
  const int nkt = (kend - kbeg + BK - 1) / BK;
  V16* lds = (V16*)smem;

  struct Regs { V16 a[A_PT]; V16 b[B_PT]; };
  auto load_tile = [&](Regs& R, int k0) {
    // unconditional loads from clamped addresses; k beyond the split is zeroed by select
#pragma unroll
    for (int p = 0; p < A_PT; ++p) {
      const int c = min(tid + p * NT, A_CH - 1);
      const int r = c / (BK / VEC), ks = c % (BK / VEC);
      const int m = min(m0 + r, a.M - 1), k = k0 + ks * VEC;
      const bool kok = k < kend;
      const V16 v = *(const V16*)((const T*)a.A + (long)a_row(a, m) * a.lda + (kok ? k : kbeg));
      R.a[p] = kok ? v : vzero();
    }
#pragma unroll
    for (int p = 0; p < B_PT; ++p) {
      const int c = min(tid + p * NT, B_CH - 1);
      const int f = c / 64, slot = c % 64;
      const int nbl = f / KCH, kcl = f % KCH;
      const int nb = min(n0 / 16 + nbl, (a.N - 1) / 16), kc = k0 / KC + kcl;
      const bool kok = kc * KC < kend;
      const V16 v = *((const V16*)a.W + ((long)nb * KB + (kok ? kc : kbeg / KC)) * 64 + slot);
      R.b[p] = kok ? v : vzero();
    }
  };
  auto store_tile = [&](const Regs& R, int stage) {
    V16* As = lds + stage * STAGE_V16;
    V16* Bs = As + A_CH;
#pragma unroll
    for (int p = 0; p < A_PT; ++p) {
      const int c = tid + p * NT;
      if (c < A_CH) {
        const int r = c / (BK / VEC), ks = c % (BK / VEC);
        As[((r / 16) * KCH + ks / SEG) * 64 + (r % 16) + 16 * (ks % SEG)] = R.a[p];
      }
    }
#pragma unroll
    for (int p = 0; p < B_PT; ++p) {
      const int c = tid + p * NT;
      if (c < B_CH) Bs[c] = R.b[p];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int stage) {
    const V16* As = lds + stage * STAGE_V16;
    const V16* Bs = As + A_CH;
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) {
      frag af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = __builtin_bit_cast(frag, As[((wm * FM + i) * KCH + kc) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = __builtin_bit_cast(frag, Bs[((wn * FN + j) * KCH + kc) * 64 + lane]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = MT::mma(af[i], bfr[j], acc[i][j]);
    }
  };

  if (a.norm != NORM_NONE) {
    RowStats<BM, NT> st;
    st.load(a, m0);
    st.merge(a, m0, s_mean, s_rinv);
  }
  Regs R0, R1;
  if (nkt > 0) load_tile(R0, kbeg);
  if (nkt > 1) load_tile(R1, kbeg + BK);
  if (nkt > 0) {
    store_tile(R0, 0);
    __syncthreads();
    for (int it = 0; it < nkt; it += 2) {
      compute(0);
      if (it + 1 < nkt) store_tile(R1, 1);
      if (it + 2 < nkt) load_tile(R0, kbeg + (it + 2) * BK);
      __syncthreads();
      if (it + 1 < nkt) {
        compute(1);
        if (it + 2 < nkt) store_tile(R0, 0);
        if (it + 3 < nkt) load_tile(R1, kbeg + (it + 3) * BK);
        __syncthreads();
      }
    }
  }

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
    constexpr int Q4 = BM * BN / 4 / NT;
    static_assert((BM * BN / 4) % NT == 0, "split items");
    const Rsrc rws = make_rsrc(a.ws, a.ws_bytes);
    const uint32_t tbase = (uint32_t)t * (uint32_t)a.splits * (BM * BN * 4);
#pragma unroll
    for (int q = 0; q < Q4; ++q) {
      const int it = tid + q * NT;
      const int r = it / (BN / 4), c4 = it % (BN / 4);
      st_dev(rws, tbase + (uint32_t)split * (BM * BN * 4) + it * 16, *(const f32x4*)(C + r * LDC + c4 * 4));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(a.counters + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)a.splits - 1u;
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int q = 0; q < Q4; ++q) {
      const int it = tid + q * NT;
      const int r = it / (BN / 4), c4 = it % (BN / 4);
      f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < a.splits; s0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = ld_dev(rws, s0 + u < a.splits ? tbase + (uint32_t)(s0 + u) * (BM * BN * 4) + it * 16 : kOob);
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
      }
      *(f32x4*)(C + r * LDC + c4 * 4) = sum;
    }
    if (tid == 0) __hip_atomic_store(a.counters + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  Epilogue<T, BM, BN, NT, EPI> ep;
  ep.prefetch(a, m0, n0);
  ep.settle();
  ep.apply(a, C, LDC, m0, n0, s_mean, s_rinv);
}

// ---------------------------------------------------------------------------------------
// Large-M kernel (bf16, K a multiple of 32): workgroup tile BM x BN (BM, BN = 128 or 256),
// WMW x WNW waves of (BM / WMW) x (BN / WNW), BK = 32 per stage. Both operand tiles are
// copied global -> LDS by buffer-to-LDS DMA in fragment-major order (the weights are
// stored that way; the activation fragments are gathered by the per-lane offsets of the
// copy), as many stages deep as the LDS budget holds (144 KB: one workgroup per CU; 64 KB
// for 128 x 128 tiles: two workgroups per CU, so that one's epilogue overlaps the other's
// main loop), so that the copies of several stages cover the memory latency. Each stage's
// fragments are all read from LDS before its MFMAs. Rows past M and columns past N read
// zeros. The epilogue runs in 64-row slabs written straight from the accumulators; split-K
// (every shape whose fp32 tile fits in the LDS budget, i.e. all but 256 x 256) exchanges
// the whole tile as in the tiled kernel.
// ---------------------------------------------------------------------------------------

// Wait until at most EXTRA + pend * PER memory operations of this wave are in flight:
// the operations issued after a stage's copies are EXTRA of its own plus PER for each of
// the pend stages issued later (pend < NST <= 6).
template <int PER, int EXTRA, int NST>
__device__ __forceinline__ void wait_stages(int pend) {
  static_assert(NST <= 6 && EXTRA + (NST - 1) * PER < 64, "vmcnt range");
  switch (pend) {
    case 5: if constexpr (NST > 5) { FM_WAIT_VM(EXTRA + 5 * PER); break; } [[fallthrough]];
    case 4: if constexpr (NST > 4) { FM_WAIT_VM(EXTRA + 4 * PER); break; } [[fallthrough]];
    case 3: if constexpr (NST > 3) { FM_WAIT_VM(EXTRA + 3 * PER); break; } [[fallthrough]];
    case 2: if constexpr (NST > 2) { FM_WAIT_VM(EXTRA + 2 * PER); break; } [[fallthrough]];
    case 1: FM_WAIT_VM(EXTRA + PER); break;
    default: FM_WAIT_VM(EXTRA); break;
  }
}

// 128 x 128 tiles of four waves run two workgroups per CU
constexpr bool big_pair(int bm, int bn, int nw) { return bm == 128 && bn == 128 && nw == 4; }

template <int BM, int BN, int NW>
struct BigShape {
  static constexpr bool PAIR = big_pair(BM, BN, NW);
  static constexpr int FS = BM / 16 + BN / 16;                // 1 KB fragments per stage
  static constexpr int BUDGET = (PAIR ? 64 : 144) * 1024;
  static constexpr int NST = BUDGET / (FS * 1024) > 6 ? 6 : BUDGET / (FS * 1024);
  static constexpr int LDC = BN + 4;
  static constexpr int OPS = NST * FS * 1024;                 // operand stages
  static constexpr int TILE = BM * LDC * 4;                   // the whole fp32 tile
  static constexpr bool WHOLE = TILE <= (PAIR ? 70 * 1024 : BUDGET);
  static constexpr int BYTES = WHOLE && TILE > OPS ? TILE : OPS;
};

template <int BM, int BN, int WMW, int WNW, int EPI, bool NORM>
__global__ void __launch_bounds__(WMW * WNW * 64, big_pair(BM, BN, WMW * WNW) ? 2 : 1) k_gemm_big(GemmArgs a) {
  typedef bf16 T;
  typedef Mma<T> MT;
  typedef typename MT::frag frag;
  typedef BigShape<BM, BN, WMW * WNW> SH;
  constexpr int NW = WMW * WNW, NT = NW * 64, VEC = MT::VEC, KC = MT::KC;
  constexpr int BK = KC;
  constexpr int RB = BM / 16, CB = BN / 16;
  constexpr int FA = RB, FB = CB, FS = FA + FB;               // 1 KB fragments per stage
  constexpr int NST = SH::NST;
  constexpr int FPW = FS / NW;
  constexpr int WRB = RB / WMW, WCB = CB / WNW;               // wave tile in 16-blocks
  constexpr int LDC = SH::LDC;
  constexpr int NSL = BM / 64;                                // 64-row epilogue slabs
  constexpr bool WHOLE = SH::WHOLE;                           // whole fp32 tile fits in LDS
  static_assert(FS % NW == 0 && RB % WMW == 0 && CB % WNW == 0 && NST >= 3, "layout");
  static_assert(64 * LDC * 4 <= SH::BYTES && (NSL % 2) == 0, "slab fits");
  __shared__ __attribute__((aligned(16))) V16 lds[SH::BYTES / 16];
  __shared__ float s_mean[BM], s_rinv[BM];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WNW, wn = w % WNW;
  const int ntn = (a.N + BN - 1) / BN, ntm = (a.M + BM - 1) / BM, tiles = ntn * ntm;
  // The grid is padded to a multiple of 8 x splits, so each XCD takes a contiguous range of
  // logical items made of whole tiles (xcd_range_item: the range of the XCD the workgroup runs
  // on): the splits of a tile are consecutive items, so they run on one XCD and exchange
  // partial tiles through its L2. Tiles are ordered in groups of 8 row tiles walked column by
  // column, so the tiles an XCD runs together share a few weight column tiles and activation
  // row tiles in its L2.
  const int bid = xcd_range_item(gridDim.x);
  if (bid >= tiles * a.splits) return;
  const int split = bid % a.splits, t = bid / a.splits;
  constexpr int GM = 8;
  const int gfirst = (t / (GM * ntn)) * GM, gsz = min(ntm - gfirst, GM);
  const int tm = gfirst + (t % (GM * ntn)) % gsz, tn = (t % (GM * ntn)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KCt = a.K / KC;
  const int kbeg = split * a.k_split;
  const int kend = min(a.K, kbeg + a.k_split);
  const int nks = (kend - kbeg) / BK;

  // this wave's copies: fragments f = w FPW + i; f < FA: A row block f, else W column
  // block f - FA. Per-copy lane offsets without the k part.
  const V16 da = make_desc(a.A, a.a_bytes), dw = make_desc(a.W, a.w_bytes);
  uint32_t coff[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int f = w * FPW + i;
    if (f < FA) {
      const int r = m0 + f * 16 + (lane % 16);
      coff[i] = r < a.M ? (uint32_t)(((long)a_row(a, r) * a.lda + (lane / 16) * VEC) * sizeof(T)) : kOob;
    } else {
      coff[i] = (uint32_t)((n0 / 16 + (f - FA)) * KCt * 1024 + lane * 16);
    }
  }
  const uint32_t lds0 = lds_addr(lds) + (uint32_t)(w * FPW) * 1024u;
  // Per copy: its buffer descriptor and the byte step per k-stage, both wave-uniform, so the
  // stage's copies issue without branches. An absent row's offset (kOob) stays past every
  // extent as it advances (K * 2 bytes < 2^31), so it needs no select.
  V16 cdesc[FPW];
  uint32_t cstep[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const bool isA = w * FPW + i < FA;
#pragma unroll
    for (int q = 0; q < 4; ++q) cdesc[i][q] = __builtin_amdgcn_readfirstlane(isA ? da[q] : dw[q]);
    cstep[i] = __builtin_amdgcn_readfirstlane(isA ? (uint32_t)(BK * sizeof(T)) : 1024u);
    coff[i] += isA ? (coff[i] == kOob ? 0u : (uint32_t)(kbeg * sizeof(T))) : (uint32_t)((kbeg / KC) * 1024);
  }
  // copies of k-stage s (relative to kbeg) into ring slot st
  auto issue = [&](int s, int st) {
#pragma unroll
    for (int i = 0; i < FPW; ++i)
      dma16_lds(cdesc[i], lds0 + (uint32_t)(st * FS + i) * 1024u, coff[i] + (uint32_t)s * cstep[i]);
  };
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < nks) issue(p, p);
  Epilogue<T, 64, BN, NT, EPI> ep0;   // per-column inputs, loaded before the main loop
  ep0.prefetch_cols(a, n0);
  if constexpr (NORM) {
    // 64-row slabs of (mu, rinv); waits here also complete the first stages
    RowStats<64, NT> st;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      st.load(a, m0 + 64 * sl);
      st.merge(a, m0 + 64 * sl, s_mean + 64 * sl, s_rinv + 64 * sl);
    }
  }

  f32x4 acc[WRB][WCB];
#pragma unroll
  for (int i = 0; i < WRB; ++i)
#pragma unroll
    for (int j = 0; j < WCB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One barrier per stage: it makes stage ks visible to every wave and also proves that
  // every wave has finished reading stage ks - 1, whose buffer the copies issued right after
  // it refill (with stage ks + NST - 1). Measured on MI355X: the steady loop without any
  // branch (no per-copy operand choice, no wait switch) is ~10% faster than with them;
  // carrying the next stage's fragments in registers during this stage's MFMAs, two stages
  // per barrier, and copies whose sources stay in cache all measured no faster.
  // Stage ks's fragments from LDS, then its MFMAs.
  auto compute = [&](int slot) {
    const V16* sA = lds + slot * FS * 64;
    const V16* sB = sA + FA * 64;
    V16 af[WRB], bfr[WCB];
#pragma unroll
    for (int i = 0; i < WRB; ++i) af[i] = sA[(wm * WRB + i) * 64 + lane];
#pragma unroll
    for (int j = 0; j < WCB; ++j) bfr[j] = sB[(wn * WCB + j) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < WRB; ++i)
#pragma unroll
      for (int j = 0; j < WCB; ++j)
        acc[i][j] = MT::mma(__builtin_bit_cast(frag, af[i]), __builtin_bit_cast(frag, bfr[j]), acc[i][j]);
  };
  // Steady state (a stage left to issue): NST - 2 later stages may still be in flight, and
  // the copies of stage ks + NST - 1 refill stage ks - 1's slot. Ring slots advance by
  // counters (NST need not be a power of two).
  int ks = 0, slot = 0, fill = NST - 1;
  for (; ks + NST - 1 < nks; ++ks) {
    FM_WAIT_VM((NST - 2) * FPW);   // stage ks has landed
    __syncthreads();
    issue(ks + NST - 1, fill);
    fill = fill + 1 == NST ? 0 : fill + 1;
    compute(slot);
    slot = slot + 1 == NST ? 0 : slot + 1;
  }
  // the last NST - 1 (or fewer) stages: nothing left to issue
  for (; ks < nks; ++ks) {
    wait_stages<FPW, 0, NST>(nks - 1 - ks);
    __syncthreads();
    compute(slot);
    slot = slot + 1 == NST ? 0 : slot + 1;
  }
  __syncthreads();   // every wave is done with the operand stages (the epilogue reuses LDS)
  float* C = (float*)lds;
  typedef Epilogue<T, 64, BN, NT, EPI> EP;
  // Row inputs (residual h, state x, RoPE cos/sin) of every slab are loaded before the
  // first store when they fit in 16 VGPR quads per thread; otherwise slab by slab.
  constexpr bool ALL = EP::ROWS && NSL * EP::ITEMS <= (EPI == EPI_QKV ? 8 : 16);
  constexpr int NEP = ALL ? NSL : 1;
  EP ep[NEP];
  ep[0].pc = ep0.pc; ep[0].pd = ep0.pd; ep[0].pb = ep0.pb; ep[0].pg = ep0.pg; ep[0].ps = ep0.ps;
#pragma unroll
  for (int e = 1; e < NEP; ++e) {
    ep[e].pc = ep0.pc; ep[e].pd = ep0.pd; ep[e].pb = ep0.pb; ep[e].pg = ep0.pg; ep[e].ps = ep0.ps;
  }
  if constexpr (ALL) {
#pragma unroll
    for (int e = 0; e < NEP; ++e) ep[e].prefetch_rows(a, m0 + 64 * e, n0);
  }
  EP::settle();   // no store of this workgroup is in flight yet

  // accumulator rows of slab sl (4 row blocks) -> C rows [0, 64) (or the whole tile)
  auto write_slab = [&](int sl, float* dst) {
#pragma unroll
    for (int i = 0; i < WRB; ++i) {
      if ((wm * WRB + i) / 4 != sl) continue;   // uniform per wave
      const int r0 = ((wm * WRB + i) % 4) * 16;
#pragma unroll
      for (int j = 0; j < WCB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[(r0 + 4 * (lane / 16) + e) * LDC + wn * WCB * 16 + j * 16 + (lane % 16)] = acc[i][j][e];
    }
  };
  // the epilogue of slab sl whose fp32 rows are at Cs
  auto apply_slab = [&](int sl, const float* Cs) {
    if constexpr (ALL) {
      ep[sl].apply(a, Cs, LDC, m0 + 64 * sl, n0, s_mean + 64 * sl, s_rinv + 64 * sl);
    } else {
      if constexpr (EP::ROWS) {
        ep[0].prefetch_rows(a, m0 + 64 * sl, n0);
        EP::settle();   // also waits for the previous slab's stores
      }
      ep[0].apply(a, Cs, LDC, m0 + 64 * sl, n0, s_mean + 64 * sl, s_rinv + 64 * sl);
    }
  };

  if constexpr (WHOLE) {
    if (a.splits > 1) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) write_slab(sl, C + 64 * sl * LDC);
      __syncthreads();
      constexpr int Q4 = BM * BN / 4 / NT;
      const Rsrc rws = make_rsrc(a.ws, a.ws_bytes);
      const uint32_t tbase = (uint32_t)t * (uint32_t)a.splits * (BM * BN * 4);
#pragma unroll 8
      for (int q = 0; q < Q4; ++q) {
        const int it = tid + q * NT;
        const int r = it / (BN / 4), c4 = it % (BN / 4);
        st_l2(rws, tbase + (uint32_t)split * (BM * BN * 4) + it * 16, *(const f32x4*)(C + r * LDC + c4 * 4));
      }
      __builtin_amdgcn_s_waitcnt(0);   // this workgroup's partial is in L2
      __syncthreads();
      if (tid == 0) s_last = l2_fetch_add(a.counters + t, 1u) == (unsigned)a.splits - 1u;
      __syncthreads();
      if (!s_last) return;
#pragma unroll 2
      for (int q = 0; q < Q4; ++q) {
        const int it = tid + q * NT;
        const int r = it / (BN / 4), c4 = it % (BN / 4);
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = ld_l2(rws, u < a.splits ? tbase + (uint32_t)u * (BM * BN * 4) + it * 16 : kOob);
        *(f32x4*)(C + r * LDC + c4 * 4) = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
      }
      if (tid == 0) l2_put(a.counters + t, 0u);
      __syncthreads();
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        if (m0 + 64 * sl >= a.M) break;   // uniform
        apply_slab(sl, C + 64 * sl * LDC);
      }
      return;
    }
  }
  // no split: slab by slab through one 64-row C buffer
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    if (m0 + 64 * sl >= a.M) break;   // uniform
    write_slab(sl, C);
    __syncthreads();
    apply_slab(sl, C);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// Skinny kernel (M <= 64, the weight-streaming regime). A workgroup covers all rows and
// 16*NB output columns over 1/splits of K (k_split), in stages of KW x CPW k-chunks: each
// wave takes CPW chunks of a stage and issues all of their loads at once, the weight
// fragments (contiguous 1 KB runs) and the matching activation fragments, through buffer
// descriptors with 32-bit offsets (rows past M and chunks past the range read zeros
// through out-of-range offsets, so nothing is clamped or selected). Two stages are in
// flight at a time. The wave partials are
// summed in LDS in wave order; with splits > 1 the workgroup partials are exchanged through
// device-scope stores and the last-arriving workgroup of the column tile sums them in split
// order before the shared epilogue. NORM: the A operand is a modulated-norm input whose row
// statistics are loaded with the operands and merged before the epilogue.
// ---------------------------------------------------------------------------------------
// ST: the range can hold more than one stage (a second register set, double buffering);
// without it the range is exactly one stage and the kernel keeps half the registers.
// W8: the weights are FP8 E4M3 codes (a.W as swizzle_fp8 lays them out: one 1 KB fragment
// holds 16 rows x 64 k, i.e. the chunk pair a wave takes per stage with CPW = 2), converted to
// bf16 exactly in registers, and the sums are scaled by the rows' powers of two before the
// epilogue. With the same chunk pairs per wave and the same split ranges as the bf16 kernel,
// the result equals the bf16 kernel's on the dequantized weights bit for bit.
// MB: 16-row blocks computed (M <= 16 MB); the tile keeps 64 rows for the epilogue and the
// statistics, and the rows past 16 MB are neither loaded, multiplied nor exchanged (at 41
// rows, three blocks instead of four: 8% less time measured on the DiT head's shapes).
template <typename T, int KW, int NB, int CPW, int MB, int EPI, bool NORM, bool ST, bool W8>
__global__ void __launch_bounds__(KW * 64) k_gemm_skinny(GemmArgs a) {
  static_assert(!W8 || (CPW == 2 && sizeof(T) == 2), "FP8 weights: chunk pairs of bf16");
  typedef Mma<T> MT;
  typedef typename MT::frag frag;
  constexpr int NT = KW * 64, VEC = MT::VEC, KC = MT::KC;
  static_assert(MB >= 1 && MB <= 4, "row blocks");
  constexpr int BM = 64, BN = 16 * NB, RI = 16 * MB * BN / 4;   // RI: 4-column items of computed rows
  constexpr int LDR = BN + 4;
  constexpr int RED = KW * BM * LDR;
  __shared__ __attribute__((aligned(16))) float red[RED];
  __shared__ float s_mean[BM], s_rinv[BM];
  __shared__ int s_last;
  // AL (bf16, chunk pairs): a wave's activations of a stage are 16 MB rows x 128 bytes (its two
  // chunks), loaded as whole rows (8 rows x 128 bytes per load: full cache lines) and turned
  // into MFMA fragments through the wave's own LDS region. Loaded as fragments, each load read
  // 16 rows x 64 bytes, which measured ~2.3 us slower per 41 x 6144 x 1536 launch from L2.
  // In LDS, row r's 16-byte piece p sits at piece p ^ ((r / 2) % 8), so that the fragment
  // reads (16 rows, one piece) and the row writes (2 rows, 8 pieces) hit 16 bank groups.
  constexpr bool AL = sizeof(T) == 2 && CPW == 2;
  __shared__ __attribute__((aligned(16))) V16 sa[AL ? KW * MB * 128 : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntn = (a.N + BN - 1) / BN;
  // The grid is padded to a multiple of 8 x splits and the splits of a column tile are
  // consecutive logical items of one XCD's range (xcd_range_item), so they run on one XCD and
  // exchange partial tiles through its L2.
  // Items are (column tile, 64-row group, split), splits innermost, then row groups, so a
  // column tile's row groups share its weights in one XCD's L2.
  const int RG = a.rgroups > 1 ? a.rgroups : 1;
  const int bid = xcd_range_item(gridDim.x);
  if (bid >= ntn * RG * a.splits) return;
  const int tr = bid / a.splits, split = bid % a.splits;   // tr: (column tile, row group)
  const int tile = tr / RG, m0 = (tr % RG) * 64;
  const int n0 = tile * BN;
  const int KCt = a.K / KC;
  // this workgroup's K range: chunks [c_lo, c_hi), walked in stages of KW x CPW chunks (wave w
  // takes CPW consecutive chunks of each stage); the next stage's loads are in flight while
  // this stage's MFMAs run
  constexpr int SPC = KW * CPW;
  const int span = a.k_split / KC;
  const int c_lo = split * span, c_hi = min(KCt, c_lo + span);
  const int nst = (c_hi - c_lo + SPC - 1) / SPC;

  // activation fragments: lane l reads row 16 mb + l % 16, k run l / 16 of every chunk
  const Rsrc ra = make_rsrc(a.A, a.a_bytes);
  uint32_t aoff[MB], arow[AL ? 2 * MB : 1];
  if constexpr (AL) {
    // row-load j: rows 8 j .. 8 j + 7, lane l takes row 8 j + l / 8 and its piece l % 8 (chunk
    // (l % 8) / 4 of the wave's pair, quarter l % 4); rows past M read row M - 1 (finite values
    // whose products land only in output rows that are never stored)
#pragma unroll
    for (int j = 0; j < 2 * MB; ++j) {
      const int r = min(m0 + 8 * j + lane / 8, a.M - 1);
      arow[j] = (uint32_t)(((long)a_row(a, r) * a.lda + (lane % 4) * VEC) * sizeof(T));
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = m0 + 16 * mb + (lane % 16);
      aoff[mb] = r < a.M ? (uint32_t)(((long)a_row(a, r) * a.lda + (lane / 16) * VEC) * sizeof(T)) : kOob;
    }
  }
  // weight fragments: fragment (nb, c) is 1 KB at ((nb * KCt + c) * 64 + lane) * 16 bytes;
  // FP8: fragment (nb, c / 2) at ((nb * KCt / 2 + c / 2) * 64 + lane) * 16 bytes
  const Rsrc rw = make_rsrc(a.W, a.w_bytes);
  const uint32_t wbase = W8 ? (uint32_t)((n0 / 16) * (KCt / 2) * 1024 + lane * 16) : (uint32_t)((n0 / 16) * KCt * 1024 + lane * 16);

  V16 ra0[CPW][MB], rb0[CPW][NB], ra1[CPW][MB], rb1[CPW][NB];
  auto issue = [&](int stg, V16 (&xa)[CPW][MB], V16 (&xb)[CPW][NB]) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int cc = c_lo + stg * SPC + w * CPW + c;
      const bool cok = cc < c_hi;   // uniform per wave
      if constexpr (AL) {
        // row-loads 2 c + {0 .. MB}: chunk min(pair start + (l % 8) / 4, last chunk) of each row;
        // a chunk outside the range multiplies zero weights
        const int ci = min(c_lo + stg * SPC + w * CPW + (lane % 8) / 4, KCt - 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xa[c][mb] = bload16(ra, arow[c * MB + mb] + (uint32_t)(ci * KC * sizeof(T)));
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xa[c][mb] = bload16(ra, cok ? aoff[mb] + (uint32_t)(cc * KC * sizeof(T)) : kOob);
      }
      if constexpr (W8) {
        // the pair's codes (chunk c_lo + ... is even: ranges and stages hold whole pairs)
        if (c == 0) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) xb[0][nb] = bload16(rw, cok ? wbase + (uint32_t)((nb * (KCt / 2) + cc / 2) * 1024) : kOob);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) xb[c][nb] = bload16(rw, cok ? wbase + (uint32_t)((nb * KCt + cc) * 1024) : kOob);
      }
    }
  };
  issue(0, ra0, rb0);
  RowStats<BM, NT> st;
  if constexpr (NORM) st.load(a, m0);
  Epilogue<T, BM, BN, NT, EPI> ep;
  ep.prefetch(a, m0, n0);
  if constexpr (ST) {
    if (nst > 1) issue(1, ra1, rb1);
  }
  // all loads are in flight before the first MFMA waits on one (the scheduler would
  // otherwise interleave them with the MFMAs and keep only a few outstanding)
  __builtin_amdgcn_sched_barrier(0);

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const V16 (&xr)[CPW][MB], const V16 (&xb)[CPW][NB]) {
    V16 xa[CPW][MB];
    if constexpr (AL) {
      // the stage's rows into this wave's region, then the fragments back out
      V16* reg = sa + w * (MB * 128);
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int j = c * MB + mb, r = 8 * j + lane / 8;
          reg[r * 8 + ((lane % 8) ^ ((r / 2) % 8))] = xr[c][mb];
        }
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xa[c][mb] = reg[(16 * mb + lane % 16) * 8 + ((c * 4 + lane / 16) ^ ((lane % 16) / 2))];
    } else {
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xa[c][mb] = xr[c][mb];
    }
    V16 wb[CPW][NB];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        wb[c][nb] = W8 ? (c == 0 ? fp8x8_bf16(xb[0][nb][0], xb[0][nb][1]) : fp8x8_bf16(xb[0][nb][2], xb[0][nb][3])) : xb[c][nb];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = MT::mma(__builtin_bit_cast(frag, xa[c][mb]), __builtin_bit_cast(frag, wb[c][nb]), acc[mb][nb]);
  };
  if constexpr (!ST) {
    mma(ra0, rb0);
  } else {
    // stages alternate between the two register sets; a set is refilled (two stages ahead)
    // right after its MFMAs have read it
    for (int stg = 0; stg < nst; stg += 2) {
      mma(ra0, rb0);
      if (stg + 2 < nst) {
        issue(stg + 2, ra0, rb0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (stg + 1 < nst) {
        mma(ra1, rb1);
        if (stg + 3 < nst) {
          issue(stg + 3, ra1, rb1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  if constexpr (NORM) st.merge(a, m0, s_mean, s_rinv);

  // wave partials -> LDS, summed in wave order
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red[(w * BM + 16 * mb + 4 * (lane / 16) + e) * LDR + 16 * nb + (lane % 16)] = acc[mb][nb][e];
  __syncthreads();
  constexpr int Q4 = (RI + NT - 1) / NT;
  f32x4 part[Q4];
#pragma unroll
  for (int q = 0; q < Q4; ++q) {
    const int i = tid + q * NT;
    part[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < RI) {
      const int r = i / (BN / 4), c4 = i % (BN / 4);
#pragma unroll
      for (int w2 = 0; w2 < KW; ++w2) part[q] += *(const f32x4*)(red + (w2 * BM + r) * LDR + c4 * 4);
    }
  }
  if (a.splits > 1) {
    const Rsrc rws = make_rsrc(a.ws, a.ws_bytes);
    const uint32_t tbase = (uint32_t)tr * (uint32_t)a.splits * (BM * BN * 4);
#pragma unroll
    for (int q = 0; q < Q4; ++q) {
      const int i = tid + q * NT;
      if (i < RI) st_l2(rws, tbase + (uint32_t)split * (BM * BN * 4) + i * 16, part[q]);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this workgroup's partial is in L2
    __syncthreads();
    if (tid == 0) s_last = l2_fetch_add(a.counters + tr, 1u) == (unsigned)a.splits - 1u;
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int q = 0; q < Q4; ++q) {
      const int i = tid + q * NT;
      if (i >= RI) continue;
      f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < a.splits; s0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = ld_l2(rws, s0 + u < a.splits ? tbase + (uint32_t)(s0 + u) * (BM * BN * 4) + i * 16 : kOob);
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
      }
      part[q] = sum;
    }
    if (tid == 0) l2_put(a.counters + tr, 0u);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < Q4; ++q) {
    const int i = tid + q * NT;
    if (i < RI) {
      const int r = i / (BN / 4), c4 = i % (BN / 4);
      if constexpr (W8) {   // the rows' scales of these four output columns (padded to N, 4)
        const int n = n0 + 4 * c4;
        part[q] *= n < a.N ? *(const f32x4*)(a.wscale + n) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      *(f32x4*)(red + r * LDR + c4 * 4) = part[q];
    }
  }
  __syncthreads();
  ep.settle();
  ep.apply(a, red, LDR, m0, n0, s_mean, s_rinv);
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
static int skinny_bn(int cfg) { return cfg == SK_N32 ? 32 : 16; }

// large-M tile shapes: cfg 0..3: bit 0 selects BN 256 (else 128), bit 1 BM 128 (else 256);
// 128 x 128 tiles run four waves, two workgroups per CU (cfg 2), or eight waves, one
// workgroup per CU (cfg 4: faster while the tiles fit in one round)
static int big_bm(int cfg) { return cfg == 4 || (cfg & 2) ? 128 : 256; }
static int big_bn(int cfg) { return cfg != 4 && (cfg & 1) ? 256 : 128; }

int gemm_num_tiles(const GemmArgs& a) {
  if (a.kind == GEMM_SKINNY) return (a.N + skinny_bn(a.cfg) - 1) / skinny_bn(a.cfg) * (a.rgroups > 1 ? a.rgroups : 1);
  if (a.kind == GEMM_BIG) return ((a.M + big_bm(a.cfg) - 1) / big_bm(a.cfg)) * ((a.N + big_bn(a.cfg) - 1) / big_bn(a.cfg));
  const CfgShape c = cfg_shape(a.cfg, ET_BF16);
  return ((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn);
}

void gemm_plan(GemmArgs& a, int elem, int num_cus) {
  const int kq = elem == ET_BF16 ? 32 : 16;
  a.fp8 = 0;       // set below where the skinny kernel streams FP8 weights
  a.rgroups = 1;   // set below where it runs over groups of 64 rows
  const int esz = elem == ET_BF16 ? 2 : 4;
  if (a.M <= 64 && elem == ET_BF16 && a.K % 32 == 0) {
    // Weight streaming in bf16: eight waves, two chunks per wave and stage (double-buffered
    // stages), 32-column tiles (the activation fragments then feed two weight columns each),
    // and a K split that brings the workgroups to about one per CU, at least 8 chunks each.
    // Measured on MI355X at 41 rows (the DiT head), against the one-stage cost model below:
    // 6144 x 1536 8.1 us (11.7), 1536 x 6144 10.1 us (13.5), 4608 x 1536 8.1 us (8.8),
    // 1536 x 1536 6.6 us (6.8); every other shape of the sweep was slower with 16 columns.
    a.kind = GEMM_SKINNY;
    a.kw = 8;
    a.cpw = 2;
    const int nb = (a.epi == EPI_RESID || a.N > 16) ? 2 : 1;
    a.cfg = nb == 2 ? SK_N32 : SK_N16;
    const int kct = a.K / kq, tiles = (a.N + 16 * nb - 1) / (16 * nb);
    int splits = num_cus / tiles;
    if (splits > kct / 8) splits = kct / 8;
    if (splits > 16) splits = 16;
    if (splits < 1) splits = 1;
    int span = (kct + splits - 1) / splits;
    // whole chunk pairs per range when K allows (the FP8 weights hold pairs; the bf16 kernel
    // takes the same ranges, so the two add the same partial sums in the same order)
    if (a.K % 64 == 0) span = (span + 1) & ~1;
    a.splits = (kct + span - 1) / span;
    a.k_split = span * kq;
    a.fp8 = a.w8 && a.wscale && a.K % 64 == 0 ? 1 : 0;
    return;
  }
  if (a.M <= 64) {
    // Weight streaming: pick the waves per workgroup (4 / 8), the column width (16 / 32),
    // the chunks per wave (2 / 4 / 8, all loaded at once) and the k-split over workgroups
    // that minimise a simple estimate: bytes each CU loads (activations are re-read by
    // every column tile) at ~105 GB/s (4 waves) or ~125 GB/s (8 waves) per CU, plus the
    // split-K exchange (a fixed round-trip cost and the last workgroup's reads of every
    // partial). Residual epilogues need whole kStatCols-column slots (32 columns).
    a.kind = GEMM_SKINNY;
    const int kct = a.K / kq;
    double best = 1e30;
    int bkw = 4, bnb = 1, bs = 1, bc = 8;
    for (int kw = 4; kw <= 8; kw *= 2) {
      if (kw == 8 && elem != ET_BF16) continue;
      for (int nb = 1; nb <= 2; ++nb) {
        if (a.epi == EPI_RESID && nb * 16 < kStatCols) continue;
        if (elem != ET_BF16 && nb > 1 && a.epi != EPI_RESID) continue;
        for (int cpw = 2; cpw <= 8; cpw *= 2) {
          if ((nb == 2 || kw == 8) && cpw > 4) continue;   // register budget
          const int per_wg = kw * cpw;
          const int splits = (kct + per_wg - 1) / per_wg;
          if (splits > 16) continue;
          const int tiles = (a.N + 16 * nb - 1) / (16 * nb);
          const int wgs = tiles * splits;
          const double kb = (double)(16 * nb + a.M) * (per_wg * kq) * esz / 1024.0;   // KB per workgroup
          const double per_cu = (double)((wgs + num_cus - 1) / num_cus) * kb;
          const double bw = kw == 8 ? 125.0 : 105.0;   // KB per microsecond per CU
          const double xchg = splits > 1 ? 2.0 + 0.02 * splits * (16 * nb * 64 * 4 / 1024.0) : 0.0;
          const double est = per_cu / bw + xchg + 0.02 * cpw;
          if (est < best) { best = est; bkw = kw; bnb = nb; bs = splits; bc = cpw; }
        }
      }
    }
    a.cfg = bnb == 2 ? SK_N32 : SK_N16;
    a.cpw = bc;
    a.kw = bkw;
    a.splits = bs;
    a.k_split = bkw * bc * kq;
    return;
  }
  if (elem == ET_BF16 && a.K % 32 == 0 && a.M <= 64 * num_cus) {
    // A few hundred rows and a narrow output: the weight-streaming kernel over 64-row groups,
    // one workgroup per (column tile, row group), when those fit in one round on the CUs (the
    // row groups of a column tile share its weights in one XCD's L2). Measured on MI355X at
    // 400 rows: 400 x 1024 x 2048 8.1 us against 17.3 for the large-M kernel, 400 x 1024 x
    // 4096 12.3 against 22.3, 400 x 2560 x 1024 (560 items, two rounds) 14.6 against 15.0
    // and 400 x 8192 x 1024 35.4 against 17.1: so only one round. 16-column tiles where they
    // also fit (not for residual epilogues, whose statistic slots are 32 columns).
    const int rg = (a.M + 63) / 64;
    const int t1 = (a.N + 15) / 16, t2 = (a.N + 31) / 32;
    const int nb = (a.epi != EPI_RESID && t1 * rg <= num_cus) ? 1 : 2;
    if ((nb == 1 ? t1 : t2) * rg <= num_cus) {
      a.kind = GEMM_SKINNY;
      a.kw = 8;
      a.cpw = 2;
      a.cfg = nb == 2 ? SK_N32 : SK_N16;
      a.rgroups = rg;
      a.splits = 1;
      a.k_split = a.K;
      a.fp8 = a.w8 && a.wscale && a.K % 64 == 0 ? 1 : 0;
      return;
    }
  }
  if (elem == ET_BF16 && a.K % 32 == 0) {
    // Large-M kernel: the tile shape and K split with the lowest estimated time. Per
    // workgroup: a fixed start (first copies, row statistics), k-stages of 32 at a
    // per-shape cost, and the epilogue; rounds of workgroups over the CUs (two per CU for
    // 128 x 128 tiles, whose stages then run slower); a split adds the partial exchange
    // (store, arrival, the last arriver's reads) and, past what the L2s hold, HBM traffic.
    // Constants measured on MI355X at M = 400 and 3200 (the pick is the fastest measured
    // choice at every expert GEMM shape).
    a.kind = GEMM_BIG;
    const int nks = a.K / 32;
    double best = 1e30;
    int bc = 0, bs = 1;
    for (int cfg = 0; cfg < 5; ++cfg) {
      if (cfg == 1 && a.epi == EPI_QKV) continue;   // its registers spill with that epilogue
      const int bm = big_bm(cfg), bn = big_bn(cfg);
      const bool pair = cfg == 2;
      const long tiles = (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
      static const double kStage[5] = {0.57, 0.95, 0.41, 0.53, 0.375};
      static const double kStart[5] = {2.8, 2.6, 1.8, 2.4, 1.8};
      static const double kEpi[5] = {4.3, 9.8, 3.8, 4.0, 3.5};
      for (int sp = 1; sp <= 8; sp *= 2) {
        if (sp > 1 && cfg == 1) break;           // the 256 x 256 fp32 tile does not fit in LDS
        if (nks / sp < 4) break;
        const int per = (nks + sp - 1) / sp;
        const int splits = (nks + per - 1) / per;
        if (splits != sp) continue;
        const long items = tiles * splits;
        const long slots = (long)num_cus * (pair ? 2 : 1);
        const long rounds = (items + slots - 1) / slots;
        const double st = pair && items > num_cus ? 0.60 : kStage[cfg];
        double est = (double)rounds * (kStart[cfg] + per * st + kEpi[cfg]);
        if (splits > 1) {
          // partial tiles go through the XCD's L2; past half of its 4 MB they spill to HBM
          const double part = (double)bm * bn * 4;
          est += 1.5 + 3.5 * part / 65536.0 + 0.8 * splits;
          const double per_xcd = (double)tiles * splits * part / 8.0;
          if (per_xcd > 2.0 * (1 << 20)) est += (per_xcd - 2.0 * (1 << 20)) * 8.0 * 2.0 / 4.0e6;
        }
        if (est < best) { best = est; bc = cfg; bs = splits; }
      }
    }
    a.cfg = bc;
    const int per = (nks + bs - 1) / bs;
    a.splits = (nks + per - 1) / per;
    a.k_split = per * 32;
    return;
  }
  a.kind = GEMM_TILED;
  if (elem == ET_BF16 && a.M >= 256 && a.N >= 512) a.cfg = GEMM_128x128;
  else a.cfg = GEMM_64x64;
  const CfgShape c = cfg_shape(a.cfg, elem);
  const int tiles = ((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn);
  const int nk = (a.K + c.bk - 1) / c.bk;
  int splits = 1;
  const int target = num_cus;
  if (tiles < target) {
    splits = (target + tiles - 1) / tiles;
    const int max_splits = nk / 4 > 0 ? nk / 4 : 1;   // at least four k-tiles per split
    if (splits > max_splits) splits = max_splits;
    if (splits > 16) splits = 16;
  }
  int kt_per = (nk + splits - 1) / splits;
  splits = (nk + kt_per - 1) / kt_per;
  a.splits = splits;
  a.k_split = kt_per * c.bk;
}

size_t gemm_ws_bytes(const GemmArgs& a) {
  if (a.splits <= 1) return 0;
  if (a.kind == GEMM_BIG) return (size_t)gemm_num_tiles(a) * a.splits * big_bm(a.cfg) * big_bn(a.cfg) * sizeof(float);
  if (a.kind == GEMM_SKINNY) return (size_t)gemm_num_tiles(a) * a.splits * 64 * skinny_bn(a.cfg) * sizeof(float);
  const CfgShape c = cfg_shape(a.cfg, ET_BF16);
  const int tiles = ((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn);
  return (size_t)tiles * a.splits * c.bm * c.bn * sizeof(float);
}

#define FM_EPI_SWITCH(KERNEL, GRID, BLOCK)                                                       \
  switch (a.epi) {                                                                             \
    case EPI_STORE: hipLaunchKernelGGL(KERNEL(EPI_STORE), GRID, BLOCK, 0, s, a); break;         \
    case EPI_GELU_MUL: hipLaunchKernelGGL(KERNEL(EPI_GELU_MUL), GRID, BLOCK, 0, s, a); break;   \
    case EPI_QKV: hipLaunchKernelGGL(KERNEL(EPI_QKV), GRID, BLOCK, 0, s, a); break;             \
    case EPI_RESID: hipLaunchKernelGGL(KERNEL(EPI_RESID), GRID, BLOCK, 0, s, a); break;         \
    case EPI_EULER: hipLaunchKernelGGL(KERNEL(EPI_EULER), GRID, BLOCK, 0, s, a); break;         \
    case EPI_VT: hipLaunchKernelGGL(KERNEL(EPI_VT), GRID, BLOCK, 0, s, a); break;               \
    default: return hipErrorInvalidValue;                                                      \
  }

template <typename T, int BM, int BN, int BK, int WM, int WN>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const dim3 grid(tiles * a.splits), block(WM * WN * 64);
#define K_TILED(E) (k_gemm<T, BM, BN, BK, WM, WN, E>)
  FM_EPI_SWITCH(K_TILED, grid, block)
#undef K_TILED
  return hipGetLastError();
}

// Skinny instantiations: the residual epilogue never consumes a norm; the others can.
template <typename T, int KW, int NB, int CPW, int MB, bool ST, bool W8>
static hipError_t launch_skinny_st(const GemmArgs& a, hipStream_t s) {
  const int per_round = 8 * a.splits;   // whole column tiles per XCD range
  const int items = ((a.N + 16 * NB - 1) / (16 * NB)) * (a.rgroups > 1 ? a.rgroups : 1) * a.splits;
  const dim3 grid((items + per_round - 1) / per_round * per_round), block(KW * 64);
  const bool norm = a.norm != NORM_NONE;
#define K_SK(E, NRM) hipLaunchKernelGGL((k_gemm_skinny<T, KW, NB, CPW, MB, E, NRM, ST, W8>), grid, block, 0, s, a)
  switch (a.epi) {
    case EPI_STORE: if (norm) K_SK(EPI_STORE, true); else K_SK(EPI_STORE, false); break;
    case EPI_GELU_MUL: if (norm) K_SK(EPI_GELU_MUL, true); else K_SK(EPI_GELU_MUL, false); break;
    case EPI_QKV: if (norm) K_SK(EPI_QKV, true); else K_SK(EPI_QKV, false); break;
    case EPI_EULER: if (norm) K_SK(EPI_EULER, true); else K_SK(EPI_EULER, false); break;
    case EPI_RESID:
      if constexpr ((16 * NB) % kStatCols == 0) {
        if (norm) return hipErrorInvalidValue;
        K_SK(EPI_RESID, false);
      } else {
        return hipErrorInvalidValue;
      }
      break;
    case EPI_VT: if (norm) return hipErrorInvalidValue; K_SK(EPI_VT, false); break;
    default: return hipErrorInvalidValue;
  }
#undef K_SK
  return hipGetLastError();
}

// a range of more than one stage needs the double-buffered kernel (CPW 2 only: registers);
// FP8 weights run with eight waves and chunk pairs only
template <typename T, int KW, int NB, int CPW>
static hipError_t launch_skinny_cpw(const GemmArgs& a, hipStream_t s) {
  const int kc = sizeof(T) == 2 ? 32 : 16;
  const bool one = a.k_split <= KW * CPW * kc;
  if constexpr (sizeof(T) == 2 && KW == 8 && CPW == 2) {
    // bf16 weight streaming: three row blocks when the rows fit (33 .. 48 rows), else four
    if (a.M <= 48) {
      if (a.fp8) return one ? launch_skinny_st<T, KW, NB, CPW, 3, false, true>(a, s) : launch_skinny_st<T, KW, NB, CPW, 3, true, true>(a, s);
      return one ? launch_skinny_st<T, KW, NB, CPW, 3, false, false>(a, s) : launch_skinny_st<T, KW, NB, CPW, 3, true, false>(a, s);
    }
    if (a.fp8) return one ? launch_skinny_st<T, KW, NB, CPW, 4, false, true>(a, s) : launch_skinny_st<T, KW, NB, CPW, 4, true, true>(a, s);
  }
  if (a.fp8) return hipErrorInvalidValue;
  if (one) return launch_skinny_st<T, KW, NB, CPW, 4, false, false>(a, s);
  if constexpr (CPW == 2) return launch_skinny_st<T, KW, NB, CPW, 4, true, false>(a, s);
  return hipErrorInvalidValue;
}

template <typename T, int KW, int NB>
static hipError_t launch_skinny_nb(const GemmArgs& a, hipStream_t s) {
  switch (a.cpw) {
    case 2: return launch_skinny_cpw<T, KW, NB, 2>(a, s);
    case 4: return launch_skinny_cpw<T, KW, NB, 4>(a, s);
    case 8:
      if constexpr (NB == 1 && KW == 4) return launch_skinny_cpw<T, KW, NB, 8>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (a.kw == 8) return a.cfg == SK_N32 ? launch_skinny_nb<T, 8, 2>(a, s) : launch_skinny_nb<T, 8, 1>(a, s);
  }
  if (a.kw != 4) return hipErrorInvalidValue;
  return a.cfg == SK_N32 ? launch_skinny_nb<T, 4, 2>(a, s) : launch_skinny_nb<T, 4, 1>(a, s);
}

template <int BM, int BN, int WMW, int WNW>
static hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
  if (a.splits > 1 && !BigShape<BM, BN, WMW * WNW>::WHOLE) return hipErrorInvalidValue;
  const int per_round = 8 * a.splits;   // whole tiles per XCD range
  const dim3 grid((gemm_num_tiles(a) * a.splits + per_round - 1) / per_round * per_round), block(WMW * WNW * 64);
  const bool norm = a.norm != NORM_NONE;
#define K_BIG(E, NRM) hipLaunchKernelGGL((k_gemm_big<BM, BN, WMW, WNW, E, NRM>), grid, block, 0, s, a)
  switch (a.epi) {
    case EPI_STORE: if (norm) K_BIG(EPI_STORE, true); else K_BIG(EPI_STORE, false); break;
    case EPI_GELU_MUL: if (norm) K_BIG(EPI_GELU_MUL, true); else K_BIG(EPI_GELU_MUL, false); break;
    case EPI_QKV: if (norm) K_BIG(EPI_QKV, true); else K_BIG(EPI_QKV, false); break;
    case EPI_EULER: if (norm) K_BIG(EPI_EULER, true); else K_BIG(EPI_EULER, false); break;
    case EPI_RESID: if (norm) return hipErrorInvalidValue; K_BIG(EPI_RESID, false); break;
    case EPI_VT: if (norm) return hipErrorInvalidValue; K_BIG(EPI_VT, false); break;
    default: return hipErrorInvalidValue;
  }
#undef K_BIG
  return hipGetLastError();
}

hipError_t gemm_launch(const GemmArgs& in, int elem, hipStream_t s) {
  if (in.M <= 0 || in.N <= 0) return hipSuccess;
  // absent optional vectors read the zeros (gate: ones) buffers; descriptor extents
  GemmArgs a = in;
  if (!a.zeros || !a.ones) return hipErrorInvalidValue;
  if (!a.cvec) a.cvec = a.zeros;
  if (!a.dvec) a.dvec = a.zeros;
  if (!a.bias) a.bias = a.zeros;
  if (!a.hscale) a.hscale = a.zeros;
  if (!a.gate) a.gate = a.ones;
  if (!a.rope_cs) a.rope_cs = (const float2*)a.zeros;
  // every vector index stays below N + 4; a substituted x / h is read over M rows
  if ((long)a.N + 4 > kVecPad) return hipErrorInvalidValue;
  if (!a.x) {
    if (a.epi == EPI_EULER && (long)a.M * a.ldo + 4 > kVecPad) return hipErrorInvalidValue;
    a.x = const_cast<float*>(a.zeros);
  }
  if (!a.h) {
    if (a.epi == EPI_RESID) return hipErrorInvalidValue;
    a.h = const_cast<float*>(a.zeros);
  }
  if (!a.stats) a.stats = (const float2*)a.zeros;
  const int esz = elem == ET_BF16 ? 2 : 4;
  const long rows = (long)((a.M - 1) / a.row_group) * a.row_gstride + a.row_off + (a.M - 1) % a.row_group + 1;
  const long a_bytes = rows * a.lda * esz;
  if (a.fp8) {
    if (a.kind != GEMM_SKINNY || elem != ET_BF16 || !a.w8 || !a.wscale || a.K % 64 != 0 || a.k_split % 64 != 0) return hipErrorInvalidValue;
    a.W = a.w8;
  }
  const long w_bytes = a.fp8 ? (long)swizzled_fp8_bytes(a.N, a.K) : (long)swizzled_bytes(a.N, a.K, elem);
  const long ws_bytes = (long)gemm_ws_bytes(a);
  if (a_bytes >= (1L << 31) || w_bytes >= (1L << 31) || ws_bytes >= (1L << 31)) return hipErrorInvalidValue;
  a.a_bytes = (uint32_t)a_bytes; a.w_bytes = (uint32_t)w_bytes; a.ws_bytes = (uint32_t)ws_bytes;
  if (a.kind == GEMM_SKINNY) {
    // more than 64 rows: bf16 row groups of 64 (rgroups of them, covering M)
    const int rg = a.rgroups > 1 ? a.rgroups : 1;
    if (a.M > 64 * rg || (rg > 1 && (elem != ET_BF16 || a.kw != 8 || a.cpw != 2))) return hipErrorInvalidValue;
    return elem == ET_BF16 ? launch_skinny<bf16>(a, s) : launch_skinny<float>(a, s);
  }
  if (a.kind == GEMM_BIG) {
    if (elem != ET_BF16 || a.K % 32 != 0 || a.splits > 8 || a.k_split % 32 != 0) return hipErrorInvalidValue;
    switch (a.cfg) {
      case 0: return launch_big<256, 128, 4, 2>(a, s);
      case 1: return launch_big<256, 256, 2, 4>(a, s);
      case 2: return launch_big<128, 128, 2, 2>(a, s);
      case 3: return launch_big<128, 256, 2, 4>(a, s);
      case 4: return launch_big<128, 128, 2, 4>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (elem == ET_BF16) {
    switch (a.cfg) {
      case GEMM_128x128: return launch_tiled<bf16, 128, 128, 64, 2, 2>(a, s);
      default: return launch_tiled<bf16, 64, 64, 64, 2, 2>(a, s);
    }
  }
  return launch_tiled<float, 64, 64, 32, 2, 2>(a, s);
}

}  // namespace fm
