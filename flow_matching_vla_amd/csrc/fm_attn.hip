// Attention of the action tokens over bound prefix / context K/V plus their own K/V
// (vla.cpp Eq. (2) with M = 0). Query rows of every head that shares a K/V head are
// folded into one row set (pi0.5 Design, "Attention and the K/V pool": the query heads
// fold onto the single K/V head), so each K/V tile is staged once in LDS and used by all
// of them.
//
// Everything is computed transposed: the score tile is S^T = K Q^T (keys as MFMA rows,
// queries as columns) and the output O^T = V^T P^T. A lane then owns one query column,
// so the softmax max and sum need only two cross-lane steps, the per-query rescale of O
// needs none, and the probabilities leave the S^T accumulators directly as the B operand
// of the P.V product, in the key order that the transposed V plane stores (vt_slot).
// K and V^T tiles are copied into LDS with buffer loads that write LDS directly (no
// register staging), double-buffered; reads past the K / V extents return zeros.
//
// A long key range can be split over workgroups; their unnormalised (O, m, l) go to a
// workspace and a second, wide kernel merges them in split order.
#include "fm_common.h"
#include "fm_kernels.h"


namespace fm {

constexpr int kKeyTile = 32;
constexpr int kAttnWaves = 8;
constexpr int kAttnRows = 16 * kAttnWaves;   // query rows per workgroup
constexpr int kMaxAttnSplits = 16;

constexpr int kAttnStages = 4;                 // LDS tile buffers (tiles in flight + 1)

// s_waitcnt with vmcnt <= n (n < 64) and the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14])
#define FM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// wait until at most `pend` tiles of FPW copies each are still in flight (pend < stages)
template <int FPW, int NST>
__device__ __forceinline__ void wait_tiles(int pend) {
  static_assert((NST - 1) * FPW < 64, "vmcnt range");
  if (pend >= 3 && NST > 3) FM_WAIT_VMCNT(3 * FPW);
  else if (pend == 2 && NST > 2) FM_WAIT_VMCNT(2 * FPW);
  else if (pend == 1) FM_WAIT_VMCNT(FPW);
  else FM_WAIT_VMCNT(0);
}

// 32-bit word with bits [0, n) set (n clamped to [0, 32])
__device__ __forceinline__ uint32_t bits_below(int n) {
  return n >= 32 ? 0xffffffffu : (n <= 0 ? 0u : (1u << n) - 1u);
}

// Element type of the key splits' partial O. Heads of 128 and 256 dims in bf16 store each
// split's O normalised by its own row sum, rounded to bf16 (the merged output is rounded to
// bf16 as well): half the bytes of the partial stores and of the merge's reads, which at
// 128 KB per 128-row tile of 256-wide heads took a large part of both launches (+3% at 8
// requests of 400 folded rows). 64-dim heads and fp32 keep the unnormalised fp32 sums.
template <typename T, int DH> struct SplitPartial { typedef float type; };
template <> struct SplitPartial<bf16, 128> { typedef bf16 type; };
template <> struct SplitPartial<bf16, 256> { typedef bf16 type; };

// WAVES waves of QB query blocks (16 rows each): ROWS = 16 WAVES QB rows per workgroup.
// Every K and V^T fragment a wave reads from LDS feeds QB MFMAs, so QB = 2 halves the LDS
// reads per MFMA (one wave per SIMD then holds twice the accumulators). VIS: the per-request
// visibility (seg_len / kmask) is applied; without it every key below n_keys is visible and
// the kernel carries none of that code (measured: the visibility code, even unused, cost
// ~10% at 64 requests).
template <typename T, int DH, int WAVES, int QB, bool VIS>
__global__ void __launch_bounds__(WAVES * 64) k_attn(AttnArgs a) {
  using MT = Mma<T>;
  typedef typename MT::frag frag;
  constexpr int VEC = MT::VEC, KC = MT::KC;
  constexpr int BK = kKeyTile;
  constexpr int KB = BK / 16, DB = DH / 16;
  constexpr int DCH = DH / KC;                 // k-chunks of S^T = K Q^T (over d)
  constexpr int KCH = BK / KC;                 // k-chunks of O^T = V^T P^T (over keys)
  constexpr int FK = KB * DCH, FV = DB * KCH;  // 1 KB fragments per K / V^T tile
  constexpr int FT = FK + FV;
  constexpr int FPW = FT / WAVES;
  constexpr int ROWS = 16 * WAVES * QB;
  static_assert(ROWS == kAttnRows, "row tile shared with the planner and the merge");
  static_assert(FT % WAVES == 0 && FPW <= 15, "tile fragments per wave");
  static_assert(KB == 2 * KCH || KB == KCH, "P fragment packing");
  constexpr int NST = kAttnStages;
  static_assert(NST >= 2 && NST <= 4, "stages");
  __shared__ __attribute__((aligned(16))) V16 sbuf[NST][FT * 64];

  // wave index made provably uniform: it selects LDS destinations (M0) of the tile copies
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.heads_per_kv * a.Tq;
  const int rtiles = (R + ROWS - 1) / ROWS;
  const int groups = a.n_heads / a.heads_per_kv;
  // Work units are (request, K/V head, key split); each unit's row tiles run on one XCD
  // (workgroup b is dispatched to XCD b mod 8) so that its K/V range is fetched from HBM
  // once and then served from that XCD's L2.
  const int units = a.B * groups * a.splits;
  const int xcd = blockIdx.x % 8, j8 = blockIdx.x / 8;
  const int unit = xcd + 8 * (j8 / rtiles);
  const int rt = j8 % rtiles;
  if (unit >= units) return;
  const int sp = unit % a.splits;
  const int g = (unit / a.splits) % groups;
  const int b = unit / (a.splits * groups);
  const int tile_id = (b * groups + g) * rtiles + rt;
  const int key_beg = sp * a.keys_per_split;
  const int key_end = min(a.n_keys, key_beg + a.keys_per_split);
  // Key tiles of this split that hold a visible key: n1 tiles from key_beg, then (with a
  // leading segment of this request's own length pb) the tiles from s2 on; the tiles in
  // between hold only keys the request does not see and are neither copied nor computed.
  typedef const __attribute__((address_space(4))) int CI;
  typedef const __attribute__((address_space(4))) uint32_t CU;
  int pb = 0x3fffffff, n1 = (key_end - key_beg + BK - 1) / BK, s2 = key_end, n2 = 0;
  if (VIS && a.seg_len) {
    pb = *(CI*)(a.seg_len + __builtin_amdgcn_readfirstlane(b));
    const int e1 = max(key_beg, min(key_end, (pb + BK - 1) / BK * BK));
    n1 = (e1 - key_beg + BK - 1) / BK;
    s2 = max(key_beg + n1 * BK, a.seg_end / BK * BK);
    n2 = key_end > s2 ? (key_end - s2 + BK - 1) / BK : 0;
  }
  const int ntile = n1 + n2;
  auto tile_start = [&](int t) { return (!VIS || t < n1) ? key_beg + t * BK : s2 + (t - n1) * BK; };

  // K / V^T tile copies: fragment f of a tile is 64 lanes x 16 bytes. K fragment (kb, c):
  // lane l carries key kb 16 + l % 16, d = c KC + (l / 16) VEC ... (A operand of S^T).
  // V^T fragment (db, kc): lane l carries d = db 16 + l % 16, stored key slots
  // kc KC + (l / 16) VEC ... (A operand of O^T). Each wave issues FPW of them per tile.
  const V16 rk = make_desc(a.k, (uint32_t)(a.k_len * (long)sizeof(T)));
  const V16 rv = make_desc(a.vt, (uint32_t)(a.v_len * (long)sizeof(T)));
  const uint32_t lds0 = lds_addr(&sbuf[0][0]) + (uint32_t)wave * FPW * 1024u;
  const uint32_t k_lane = (uint32_t)(((long)b * a.k_bs + (long)g * a.k_hs + (long)(lane % 16) * a.k_rs + (lane / 16) * VEC) * sizeof(T));
  const uint32_t v_lane = (uint32_t)(((long)b * a.v_bs + (long)g * a.v_hs + (long)(lane % 16) * a.v_ds + (lane / 16) * VEC) * sizeof(T));
  const uint32_t k_row = (uint32_t)(a.k_rs * sizeof(T)), v_row16 = (uint32_t)(16 * a.v_ds * sizeof(T));
  // Per copy: its descriptor, its lane offset at key 0 and its bytes per key, all but the
  // lane offset wave-uniform, so a tile's copies issue without branches.
  V16 cdesc[FPW];
  uint32_t cbase[FPW], cper[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int f = wave * FPW + i;
    const bool isK = f < FK;
    const int kb = f / DCH, c = f % DCH, fv = f - FK, db = fv / KCH, kc = fv % KCH;
#pragma unroll
    for (int q = 0; q < 4; ++q) cdesc[i][q] = __builtin_amdgcn_readfirstlane(isK ? rk[q] : rv[q]);
    cbase[i] = isK ? k_lane + (uint32_t)(16 * kb) * k_row + (uint32_t)(c * KC * sizeof(T))
                   : v_lane + (uint32_t)db * v_row16 + (uint32_t)(kc * KC * sizeof(T));
    cper[i] = __builtin_amdgcn_readfirstlane(isK ? k_row : (uint32_t)sizeof(T));
  }
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < FPW; ++i)
      dma16_lds(cdesc[i], lds0 + (uint32_t)buf * (FT * 1024u) + i * 1024u, cbase[i] + (uint32_t)kt * cper[i]);
  };
  if (ntile > 0) issue(tile_start(0), 0);   // tile 0 first, the other prefetched tiles after Q

  // Q^T fragments (B operand of S^T): lane l carries query row l % 16 of query block
  // wave QB + qb, d run l / 16 of every d-chunk. Rows past R read row R-1; their outputs
  // are not stored.
  frag qf[QB][DCH];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = min(rt * ROWS + (wave * QB + qb) * 16 + (lane % 16), R - 1);
    const int n = g * a.heads_per_kv + r / a.Tq, t = r % a.Tq;
    const T* qp = (const T*)a.q + (long)b * a.q_bs + (long)t * a.q_rs + (long)n * a.dh + (lane / 16) * VEC;
#pragma unroll
    for (int c = 0; c < DCH; ++c) qf[qb][c] = __builtin_bit_cast(frag, *(const V16*)(qp + c * KC));
  }
  // Q and the first tile's copies complete here; the loop below then waits only on the
  // copies it issues itself (the compiler cannot see those: they are inline asm)
  FM_WAIT_VMCNT(0);
#pragma unroll
  for (int p = 1; p < NST - 1; ++p)
    if (p < ntile) issue(tile_start(p), p);

  f32x4 o[QB][DB];   // O^T: lane l, element e holds d = 16 db + 4 (l / 16) + e of query l % 16
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < DB; ++i) o[qb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // of this lane's queries, base-2 logits. The reference starts finite (below any score),
  // so a tile whose keys this query cannot see gives weights exp2(-inf - m) = 0, and a split
  // with none leaves (O, l) = 0 and a reference the merge weighs by exp2(-1e30 - m) = 0.
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = VIS ? -1e30f : -INFINITY; l_run[qb] = 0.f; }

  // a wave whose query rows all lie past R (the row tile's unused tail, e.g. 41 DiT tokens in
  // a 128-row tile) still copies its share of every tile and meets every barrier, but reads
  // no fragment and computes nothing (wave-uniform)
  const bool active = rt * ROWS + wave * QB * 16 < R;
  // One barrier per tile: after it, tile t is visible to every wave and every wave has left
  // tile t - 1, whose buffer then takes tile t + NST - 1 (the copies run during the compute).
  for (int t = 0; t < ntile; ++t) {
    const int kt = tile_start(t);
    // visibility bits of the tile's 32 keys (a scalar load: its wait does not count the
    // tile copies)
    uint32_t vis = 0xffffffffu;
    if constexpr (VIS) {
      if (a.kmask) vis = *(CU*)(a.kmask + __builtin_amdgcn_readfirstlane((int)(b * a.km_bs) + (kt >> 5)));
      // bit i of vis: key kt + i is visible (uniform: scalar arithmetic)
      vis &= bits_below(key_end - kt);
      vis &= ~(bits_below(a.seg_end - kt) & ~bits_below(pb - kt));   // the keys in [pb, seg_end)
    }
    // tile t's copies are done once at most the tiles issued after it (t + 1 .. t + NST - 2)
    // are in flight
    if (t + NST - 2 < ntile) FM_WAIT_VMCNT((NST - 2) * FPW);
    else wait_tiles<FPW, NST>(ntile - 1 - t);
    __syncthreads();
    if (t + NST - 1 < ntile) issue(tile_start(t + NST - 1), (t + NST - 1) % NST);
    const V16* sK = sbuf[t % NST];
    const V16* sV = sK + FK * 64;
    if (active) {

    // S^T = K Q^T: 16 keys x 16 queries per (kb, qb), two partial chains each. A key
    // block's fragments are all read from LDS before its MFMAs, so the reads overlap each
    // other instead of each MFMA waiting on its own read.
    f32x4 s[QB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      V16 kf[DCH];
#pragma unroll
      for (int c = 0; c < DCH; ++c) kf[c] = sK[(kb * DCH + c) * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
        for (int c = 0; c < DCH; c += 2) {
          s0 = MT::mma(__builtin_bit_cast(frag, kf[c]), qf[qb][c], s0);
          if (c + 1 < DCH) s1 = MT::mma(__builtin_bit_cast(frag, kf[c + 1]), qf[qb][c + 1], s1);
        }
        s[qb][kb] = s0 + s1;
      }
    }
    // V^T fragments read now; their LDS latency hides behind the softmax
    V16 vf[FV];
#pragma unroll
    for (int f = 0; f < FV; ++f) vf[f] = sV[f * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
    // online softmax of this lane's queries over keys kt + 16 kb + 4 (l / 16) + e; a tile
    // whose keys are all visible (the common case) skips the per-key test
    const uint32_t lvis = vis >> (4 * (lane / 16));
    frag pf[QB][KCH];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mt = -INFINITY;
      if constexpr (!VIS) {
        const int kl = kt + 4 * (lane / 16);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = (kl + 16 * kb + e < key_end) ? s[qb][kb][e] * a.scale_log2 : -INFINITY;
            s[qb][kb][e] = v;
            mt = fmaxf(mt, v);
          }
      } else if (vis == 0xffffffffu) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[qb][kb][e] *= a.scale_log2;
            mt = fmaxf(mt, s[qb][kb][e]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = ((lvis >> (16 * kb + e)) & 1u) ? s[qb][kb][e] * a.scale_log2 : -INFINITY;
            s[qb][kb][e] = v;
            mt = fmaxf(mt, v);
          }
      }
      mt = group4_max(mt);
      // The reference max moves only when a score exceeds it by more than 2^8: until then
      // p = 2^(s - m_run) <= 256 stays exact in fp32 / bf16 and O, l need no rescale. The
      // final O / l is the same for any reference, so this changes no result.
      if (__builtin_amdgcn_ballot_w64(mt > m_run[qb] + 8.f)) {   // wave-uniform
        const float m_new = fmaxf(m_run[qb], mt);
        const float alpha = exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[qb][i] *= alpha;
      }
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2f(s[qb][kb][e] - m_run[qb]);
          s[qb][kb][e] = p;
          ls += p;
        }
      ls = group4_sum(ls);
      l_run[qb] += ls;
      // P^T fragments: keys 16 h + 4 (l / 16) + r of chunk kc, h over the chunk's key blocks
#pragma unroll
      for (int kc = 0; kc < KCH; ++kc) {
        if constexpr (sizeof(T) == 2) {
          const f32x4 p0 = s[qb][2 * kc], p1 = s[qb][2 * kc + 1];
          pf[qb][kc] = frag{(bf16)p0[0], (bf16)p0[1], (bf16)p0[2], (bf16)p0[3], (bf16)p1[0], (bf16)p1[1], (bf16)p1[2], (bf16)p1[3]};
        } else {
          pf[qb][kc] = __builtin_bit_cast(frag, s[qb][kc]);
        }
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = MT::mma(__builtin_bit_cast(frag, vf[db * KCH + kc]), pf[qb][kc], o[qb][db]);
    }
  }

  if (a.splits == 1) {
    // The normalised output goes through LDS so that every global store writes whole rows:
    // a lane's MFMA-layout values are four d of one row, and stored directly each store
    // instruction wrote 16 rows x 32 bytes (measured ~5 us of a 57 us launch at 64 requests).
    // Rows are padded by 16 bytes, so the row-per-lane writes hit distinct banks.
    constexpr int RBY = DH * (int)sizeof(T), RST = RBY + 16, CPR = RBY / 16;
    static_assert(WAVES * QB * 16 * RST <= NST * FT * 1024, "output staging fits the tile buffers");
    __syncthreads();   // every wave is done with the last tile's buffer
    char* st = (char*)&sbuf[0][0] + (size_t)wave * QB * 16 * RST;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float inv = 1.f / l_run[qb];
      char* rowp = st + (qb * 16 + lane % 16) * RST + 4 * (lane / 16) * (int)sizeof(T);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (sizeof(T) == 2) {
          *(bf16x4*)(rowp + db * 32) = bf16x4{(bf16)(o[qb][db][0] * inv), (bf16)(o[qb][db][1] * inv), (bf16)(o[qb][db][2] * inv), (bf16)(o[qb][db][3] * inv)};
        } else {
          *(f32x4*)(rowp + db * 64) = o[qb][db] * inv;
        }
      }
    }
    // each lane then stores 16-byte chunks of whole rows
#pragma unroll
    for (int i = 0; i < QB * 16 * CPR / 64; ++i) {
      const int c = i * 64 + lane, rl = c / CPR, ch = c % CPR;
      const int rq = rt * ROWS + wave * QB * 16 + rl;
      const V16 v = *(const V16*)(st + rl * RST + ch * 16);
      if (rq < R) {
        const int n = g * a.heads_per_kv + rq / a.Tq, t = rq % a.Tq;
        *(V16*)((char*)((T*)a.o + (long)b * a.o_bs + (long)t * a.o_rs + (long)n * a.dh) + ch * 16) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int blk = wave * QB + qb;                      // 16-row block of the row tile
    // split keys: O^T (SplitPartial: unnormalised fp32, or normalised by the split's own row
    // sum in bf16) in the MFMA output layout ([block][db][lane][e], one store per lane and
    // d-block), and (m, l) of each query row; a split that sees none of a row's keys (l = 0)
    // stores zeros, which the merge weighs by l = 0. An inactive wave's rows are past R, and
    // the merge never stores them.
    if (!active) continue;
    typedef typename SplitPartial<T, DH>::type P;
    P* wo = (P*)a.ws + ((long)tile_id * a.splits + sp) * (ROWS * DH);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      P* p = wo + ((blk * DB + db) * 64 + lane) * 4;
      if constexpr (sizeof(P) == 2) {
        const float inv = l_run[qb] > 0.f ? 1.f / l_run[qb] : 0.f;
        *(bf16x4*)p = bf16x4{(bf16)(o[qb][db][0] * inv), (bf16)(o[qb][db][1] * inv), (bf16)(o[qb][db][2] * inv), (bf16)(o[qb][db][3] * inv)};
      } else {
        *(f32x4*)p = o[qb][db];
      }
    }
    if (lane < 16) {
      float2* wml = (float2*)((P*)a.ws + (long)a.B * groups * rtiles * a.splits * (ROWS * DH)) + ((long)tile_id * a.splits + sp) * ROWS;
      wml[blk * 16 + lane] = make_float2(m_run[qb], l_run[qb]);
    }
  }
}

// Merge of the key splits: thread = (row tile, wave, d-block, lane) of the partial layout,
// i.e. four consecutive d of one query row. All NS (>= splits) partials and (m, l) pairs
// are loaded before any is used (clamped split index, weight 0 past the split count).
template <typename T, int DH, int ROWS, int NS>
__global__ void __launch_bounds__(256) k_attn_combine(AttnArgs a) {
  constexpr int DB = DH / 16, PER_TILE = ROWS * DH / 4;
  const int R = a.heads_per_kv * a.Tq;
  const int rtiles = (R + ROWS - 1) / ROWS;
  const int groups = a.n_heads / a.heads_per_kv;
  const long ntiles = (long)a.B * groups * rtiles;
  const long it = blockIdx.x * 256L + threadIdx.x;
  if (it >= ntiles * PER_TILE) return;
  const int tile_id = (int)(it / PER_TILE), w = (int)(it % PER_TILE);
  const int lane = w % 64, db = (w / 64) % DB, wave = w / (64 * DB);
  const int rt = tile_id % rtiles, g = (tile_id / rtiles) % groups, b = tile_id / (rtiles * groups);
  const int rl = wave * 16 + (lane % 16);
  const int r = rt * ROWS + rl;
  if (r >= R) return;   // a row tile's tail past R: its partials were never stored
  const int S = a.splits;
  typedef typename SplitPartial<T, DH>::type P;
  const P* wo = (const P*)a.ws + (long)tile_id * S * (ROWS * DH) + (long)w * 4;
  const float2* wml = (const float2*)((const P*)a.ws + ntiles * S * (ROWS * DH)) + (long)tile_id * S * ROWS + rl;
  f32x4 ov[NS];
  float2 ml[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int sc = min(s, S - 1);
    if constexpr (sizeof(P) == 2) {
      const bf16x4 v = *(const bf16x4*)(wo + (long)sc * (ROWS * DH));
      ov[s] = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    } else {
      ov[s] = *(const f32x4*)(wo + (long)sc * (ROWS * DH));
    }
    ml[s] = wml[(long)sc * ROWS];
  }
  float mx = ml[0].x;
#pragma unroll
  for (int s = 1; s < NS; ++s) mx = fmaxf(mx, ml[s].x);   // clamped copies repeat a real split
  // a normalised partial weighs by its split's share of the row's exponential sum
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float e = s < S ? exp2f(ml[s].x - mx) : 0.f;
    const float wgt = sizeof(P) == 2 ? e * ml[s].y : e;
    num += wgt * ov[s];
    den += e * ml[s].y;
  }
  const int n = g * a.heads_per_kv + r / a.Tq, t = r % a.Tq;
  T* op = (T*)a.o + (long)b * a.o_bs + (long)t * a.o_rs + (long)n * a.dh + db * 16 + 4 * (lane / 16);
  const float inv = 1.f / den;
  if constexpr (sizeof(T) == 2) {
    *(bf16x4*)op = bf16x4{(bf16)(num[0] * inv), (bf16)(num[1] * inv), (bf16)(num[2] * inv), (bf16)(num[3] * inv)};
  } else {
    *(f32x4*)op = num * inv;
  }
}

int attn_num_items(const AttnArgs& a) {
  const int R = a.heads_per_kv * a.Tq;
  return a.B * (a.n_heads / a.heads_per_kv) * ((R + kAttnRows - 1) / kAttnRows);
}

void attn_plan(AttnArgs& a, int elem, int num_cus) {
  // Split the keys when the row tiles alone leave part of the chip idle. The merge reads
  // every split's partial O (4 bytes per row and head dim), so splits keep at least two key
  // tiles, and the launch aims at one workgroup per CU (measured at 8 requests of 400 folded
  // rows and 866 keys: 34 us per layer at a quarter of the CUs, 26 at half, 25.8 at all;
  // never splitting short key ranges was much slower: 48 us there, 14 against 10.6 us for
  // the DiT head's 600-key cross attention).
  a.cfg = 0;
  const int items = attn_num_items(a);
  const int ktiles = (a.n_keys + kKeyTile - 1) / kKeyTile;
  int splits = 1;
  const int target = num_cus > 0 ? num_cus : 1;
  if (items < target) {
    splits = (target + items - 1) / items;
    const int max_splits = ktiles / 2 > 1 ? ktiles / 2 : 1;
    if (splits > max_splits) splits = max_splits;
    if (splits > kMaxAttnSplits) splits = kMaxAttnSplits;
  }
  const int per = (ktiles + splits - 1) / splits;
  a.splits = (ktiles + per - 1) / per;
  a.keys_per_split = per * kKeyTile;
  (void)elem;
}

// sized for fp32 partials (bf16 ones use half of the first part)
size_t attn_ws_bytes(const AttnArgs& a) {
  if (a.splits <= 1) return 0;
  return (size_t)attn_num_items(a) * a.splits * ((size_t)kAttnRows * a.dh + 2 * kAttnRows) * sizeof(float);
}

template <typename T, int DH>
static void launch_attn(const AttnArgs& a, hipStream_t s) {
  const int R = a.heads_per_kv * a.Tq;
  const int rtiles = (R + kAttnRows - 1) / kAttnRows;
  const int units = a.B * (a.n_heads / a.heads_per_kv) * a.splits;
  const dim3 grid(8 * ((units + 7) / 8) * rtiles);
  // one query block per wave: two blocks per wave (four waves, one per SIMD) halve the LDS
  // reads per MFMA but measured slower (pi05_b64: 73 against 62 us per layer), the single
  // wave per SIMD leaving LDS and softmax latencies uncovered
  if (a.seg_len || a.kmask) hipLaunchKernelGGL((k_attn<T, DH, kAttnWaves, 1, true>), grid, dim3(64 * kAttnWaves), 0, s, a);
  else hipLaunchKernelGGL((k_attn<T, DH, kAttnWaves, 1, false>), grid, dim3(64 * kAttnWaves), 0, s, a);
  if (a.splits > 1) {
    const long threads = (long)attn_num_items(a) * kAttnRows * DH / 4;
    const dim3 cgrid((unsigned)((threads + 255) / 256));
    if (a.splits <= 4) hipLaunchKernelGGL((k_attn_combine<T, DH, kAttnRows, 4>), cgrid, dim3(256), 0, s, a);
    else if (a.splits <= 8) hipLaunchKernelGGL((k_attn_combine<T, DH, kAttnRows, 8>), cgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_attn_combine<T, DH, kAttnRows, 16>), cgrid, dim3(256), 0, s, a);
  }
}

hipError_t attn_launch(const AttnArgs& a, int elem, hipStream_t s) {
  if (attn_num_items(a) == 0) return hipSuccess;
  if (a.splits < 1 || a.splits > kMaxAttnSplits || a.keys_per_split % kKeyTile != 0) return hipErrorInvalidValue;
  // K / V^T are addressed through 32-bit byte offsets
  const long esz = elem == ET_BF16 ? 2 : 4;
  if (a.k_len <= 0 || a.v_len <= 0 || a.k_len * esz >= (1L << 31) || a.v_len * esz >= (1L << 31)) return hipErrorInvalidValue;
  if (elem == ET_BF16) {
    if (a.dh == 256) launch_attn<bf16, 256>(a, s);
    else if (a.dh == 64) launch_attn<bf16, 64>(a, s);
    else if (a.dh == 128) launch_attn<bf16, 128>(a, s);
    else return hipErrorInvalidValue;
  } else {
    if (a.dh == 64) launch_attn<float, 64>(a, s);
    else if (a.dh == 128) launch_attn<float, 128>(a, s);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fm
