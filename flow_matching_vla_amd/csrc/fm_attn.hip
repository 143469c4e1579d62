// Attention of the action tokens over bound prefix / context K/V plus their own K/V
// (vla.cpp Eq. (2) with M = 0). Query rows of every head that shares a K/V head are
// folded into one row set (pi0.5 Design, "Attention and the K/V pool": the query heads
// fold onto the single K/V head), so each K/V tile is staged once in LDS and used by all
// of them. Scores and P.V run on MFMA; the softmax is computed online with wave-level
// row reductions; a long key range can be split over workgroups, whose partial (O, m, l)
// are merged in split order by the last workgroup of the row tile. V is read from a
// transposed layout (key index contiguous) so both products take 16-byte fragments.
#include "fm_common.h"
#include "fm_kernels.h"

namespace fm {

constexpr int kKeyTile = 64;

template <typename T, int DH, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) k_attn(AttnArgs a) {
  using MT = Mma<T>;
  typedef typename MT::frag frag;
  constexpr int NT = WAVES * 64;
  constexpr int VEC = MT::VEC, KC = MT::KC, SEG = KC / VEC;
  constexpr int BK = kKeyTile;
  constexpr int DCH = DH / KC;                 // d-chunks (QK^T reduction)
  constexpr int KCH = BK / KC;                 // key-chunks (PV reduction)
  constexpr int KB = BK / 16, DB = DH / 16;
  constexpr int K_V16 = BK * DH / VEC;         // 16-byte chunks per K (and per V) tile
  constexpr int P_V16 = 16 * BK / VEC;         // per wave
  constexpr int ROWS = 16 * WAVES;
  __shared__ __attribute__((aligned(16))) V16 sK[K_V16];
  __shared__ __attribute__((aligned(16))) V16 sV[K_V16];
  __shared__ __attribute__((aligned(16))) V16 sP[WAVES * P_V16];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.heads_per_kv * a.Tq;
  const int rtiles = (R + ROWS - 1) / ROWS;
  const int groups = a.n_heads / a.heads_per_kv;
  const int item = xcd_swizzle(blockIdx.x, gridDim.x);
  const int sp = item % a.splits;
  const int tile_id = item / a.splits;          // (b, g, rt)
  const int rt = tile_id % rtiles;
  const int g = (tile_id / rtiles) % groups;
  const int b = tile_id / (rtiles * groups);
  const int key_beg = sp * a.keys_per_split;
  const int key_end = min(a.n_keys, key_beg + a.keys_per_split);

  const T* kbase = (const T*)a.k + (long)b * a.k_bs + (long)g * a.k_hs;
  const T* vbase = (const T*)a.vt + (long)b * a.v_bs + (long)g * a.v_hs;

  // this lane's query row for the Q fragments
  // (loads are unconditional from clamped addresses: rows past R produce outputs that are
  // never stored, keys past the range are masked in the softmax and zeroed in V)
  frag qf[DCH];
  {
    const int r = min(rt * ROWS + wave * 16 + (lane % 16), R - 1);
    const int n = g * a.heads_per_kv + r / a.Tq, t = r % a.Tq;
    const T* qp = (const T*)a.q + (long)b * a.q_bs + (long)t * a.q_rs + (long)n * a.dh + (lane / 16) * VEC;
#pragma unroll
    for (int c = 0; c < DCH; ++c) qf[c] = __builtin_bit_cast(frag, *(const V16*)(qp + c * KC));
  }

  f32x4 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { mrow[e] = -INFINITY; lrow[e] = 0.f; }

  T* pw = (T*)(sP + wave * P_V16);

  // K / V^T tiles: the next tile's global loads are issued before the current tile's MFMA
  // work, so one memory round trip per tile is hidden behind compute.
  constexpr int KPT = (K_V16 + NT - 1) / NT;
  V16 rk[KPT], rv[KPT];
  auto load_kv = [&](int kt) {
    const int jlast = ((key_end - 1) / VEC) * VEC;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int c = min(tid + q * NT, K_V16 - 1);
      const int j = c / (DH / VEC), ds = c % (DH / VEC);
      rk[q] = *(const V16*)(kbase + (long)min(kt + j, key_end - 1) * a.k_rs + ds * VEC);
      const int d = c / (BK / VEC), ks = c % (BK / VEC);
      const int j0 = kt + ks * VEC;
      V16 v = *(const V16*)(vbase + (long)d * a.v_ds + min(j0, jlast));
      const int nv = key_end - j0;  // keys of this chunk inside the range (may be <= 0)
      constexpr int EPW = VEC / 4;  // elements per 32-bit word
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e0 = w * EPW;
        const uint32_t keep = (e0 + EPW <= nv) ? 0xffffffffu : (e0 < nv ? 0x0000ffffu : 0u);
        v[w] &= keep;
      }
      rv[q] = v;
    }
  };
  auto store_kv = [&]() {
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int c = tid + q * NT;
      if (c < K_V16) {
        const int j = c / (DH / VEC), ds = c % (DH / VEC);
        sK[((j / 16) * DCH + ds / SEG) * 64 + (j % 16) + 16 * (ds % SEG)] = rk[q];
        const int d = c / (BK / VEC), ks = c % (BK / VEC);
        sV[((d / 16) * KCH + ks / SEG) * 64 + (d % 16) + 16 * (ks % SEG)] = rv[q];
      }
    }
  };

  if (key_beg < key_end) load_kv(key_beg);
  for (int kt = key_beg; kt < key_end; kt += BK) {
    store_kv();
    __syncthreads();
    if (kt + BK < key_end) load_kv(kt + BK);

    // S = Q K^T for 16 rows x BK keys
    f32x4 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DCH; ++c)
        s[kb] = MT::mma(qf[c], __builtin_bit_cast(frag, sK[(kb * DCH + c) * 64 + lane]), s[kb]);
    }
    // online softmax (base 2): lane holds rows 4 (l/16) + e, key 16 kb + l % 16
    float mt[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) mt[e] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bool valid = kt + kb * 16 + (lane % 16) < key_end;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = valid ? s[kb][e] * a.scale_log2 : -INFINITY;
        s[kb][e] = v;
        mt[e] = fmaxf(mt[e], v);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      for (int off = 1; off < 16; off <<= 1) mt[e] = fmaxf(mt[e], __shfl_xor(mt[e], off, 64));
    float alpha[4], ls[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mn = fmaxf(mrow[e], mt[e]);
      alpha[e] = exp2f(mrow[e] - mn);
      mrow[e] = mn;
      ls[e] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = exp2f(s[kb][e] - mrow[e]);
        s[kb][e] = p;
        ls[e] += p;
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      for (int off = 1; off < 16; off <<= 1) ls[e] += __shfl_xor(ls[e], off, 64);
      lrow[e] = lrow[e] * alpha[e] + ls[e];
    }
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[i][e] *= alpha[e];
    // P -> LDS in A-fragment order: element (row r, key c) of chunk c / KC
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * (lane / 16) + e, c = kb * 16 + (lane % 16);
        const int slot = r + 16 * ((c % KC) / VEC);
        pw[((c / KC) * 64 + slot) * VEC + (c % VEC)] = from_f32<T>(s[kb][e]);
      }
    __syncthreads();
    // O += P V
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) {
      const frag pf = __builtin_bit_cast(frag, sP[wave * P_V16 + kc * 64 + lane]);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = MT::mma(pf, __builtin_bit_cast(frag, sV[(db * KCH + kc) * 64 + lane]), o[db]);
    }
    __syncthreads();
  }

  const int row0 = rt * ROWS + wave * 16 + 4 * (lane / 16);
  if (a.splits == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = row0 + e;
      if (r >= R) continue;
      const int n = g * a.heads_per_kv + r / a.Tq, t = r % a.Tq;
      T* op = (T*)a.o + (long)b * a.o_bs + (long)t * a.o_rs + (long)n * a.dh;
      const float inv = 1.f / lrow[e];
#pragma unroll
      for (int db = 0; db < DB; ++db) op[db * 16 + (lane % 16)] = from_f32<T>(o[db][e] * inv);
    }
    return;
  }

  // split keys: partial (O, m, l) to the workspace with device-scope stores (coherent
  // across XCDs without an L2 write-back); the last arriver merges them in split order
  const long per = (long)ROWS * DH + 2L * ROWS;
  float* wt = a.ws + (long)tile_id * a.splits * per;
  {
    float* wo = wt + (long)sp * per;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = wave * 16 + 4 * (lane / 16) + e;
#pragma unroll
      for (int db = 0; db < DB; ++db) st_dev1(wo + (long)rl * DH + db * 16 + (lane % 16), o[db][e]);
      if ((lane % 16) == 0) {
        st_dev1(wo + (long)ROWS * DH + rl, mrow[e]);
        st_dev1(wo + (long)ROWS * DH + ROWS + rl, lrow[e]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(a.counters + tile_id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)a.splits - 1u;
  __syncthreads();
  if (!s_last) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int rl = wave * 16 + 4 * (lane / 16) + e;
    const int r = rt * ROWS + rl;
    float mx = -INFINITY;
    for (int q0 = 0; q0 < a.splits; q0 += 8) {
      float mv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float m_u = ld_dev1(wt + (long)min(q0 + u, a.splits - 1) * per + (long)ROWS * DH + rl);
        mv[u] = q0 + u < a.splits ? m_u : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) mx = fmaxf(mx, mv[u]);
    }
    float den = 0.f;
    float acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = 0.f;
    for (int q0 = 0; q0 < a.splits; q0 += 2) {
      float w[2], lv[2], ov[2][DB];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool ok = q0 + u < a.splits;
        const float* wq = wt + (long)(ok ? q0 + u : 0) * per;
        const float m_u = ld_dev1(wq + (long)ROWS * DH + rl);
        w[u] = ok ? m_u : -INFINITY;
        lv[u] = ld_dev1(wq + (long)ROWS * DH + ROWS + rl);
#pragma unroll
        for (int db = 0; db < DB; ++db) ov[u][db] = ld_dev1(wq + (long)rl * DH + db * 16 + (lane % 16));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float wt_u = exp2f(w[u] - mx);
        den += wt_u * lv[u];
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] += wt_u * ov[u][db];
      }
    }
    if (r < R) {
      const int n = g * a.heads_per_kv + r / a.Tq, t = r % a.Tq;
      T* op = (T*)a.o + (long)b * a.o_bs + (long)t * a.o_rs + (long)n * a.dh;
      const float inv = 1.f / den;
#pragma unroll
      for (int db = 0; db < DB; ++db) op[db * 16 + (lane % 16)] = from_f32<T>(acc[db] * inv);
    }
  }
  if (tid == 0) __hip_atomic_store(a.counters + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static int attn_rows(int elem, int dh) { (void)elem; (void)dh; return 64; }

int attn_num_items(const AttnArgs& a) {
  const int rows = attn_rows(0, a.dh);
  const int R = a.heads_per_kv * a.Tq;
  return a.B * (a.n_heads / a.heads_per_kv) * ((R + rows - 1) / rows);
}

void attn_plan(AttnArgs& a, int elem, int num_cus) {
  a.cfg = 0;
  const int items = attn_num_items(a);
  const int ktiles = (a.n_keys + kKeyTile - 1) / kKeyTile;
  int splits = 1;
  if (items < num_cus) {
    splits = (num_cus + items - 1) / items;
    if (splits > ktiles) splits = ktiles;
  }
  const int per = (ktiles + splits - 1) / splits;
  a.splits = (ktiles + per - 1) / per;
  a.keys_per_split = per * kKeyTile;
  (void)elem;
}

size_t attn_ws_bytes(const AttnArgs& a) {
  if (a.splits <= 1) return 0;
  const int rows = attn_rows(0, a.dh);
  return (size_t)attn_num_items(a) * a.splits * ((size_t)rows * a.dh + 2 * rows) * sizeof(float);
}

hipError_t attn_launch(const AttnArgs& a, int elem, hipStream_t s) {
  const dim3 grid(attn_num_items(a) * a.splits), block(256);
  if (grid.x == 0) return hipSuccess;
  if (elem == ET_BF16) {
    if (a.dh == 256) hipLaunchKernelGGL((k_attn<bf16, 256, 4>), grid, block, 0, s, a);
    else if (a.dh == 64) hipLaunchKernelGGL((k_attn<bf16, 64, 4>), grid, block, 0, s, a);
    else if (a.dh == 128) hipLaunchKernelGGL((k_attn<bf16, 128, 4>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    if (a.dh == 64) hipLaunchKernelGGL((k_attn<float, 64, 4>), grid, block, 0, s, a);
    else if (a.dh == 128) hipLaunchKernelGGL((k_attn<float, 128, 4>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fm
