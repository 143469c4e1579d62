// Persistent denoise loop for the weight-streaming regime (one request batch of at most 64
// action rows, pi0.5-shaped expert, bf16): every Euler step of a chunk runs inside ONE
// cooperative launch of one workgroup per CU. The step is a chain of phases
//   in-projection, then per layer: QKV + RoPE (+ suffix K/V), attention partials over key
//   splits, split merge, O projection + gated residual, gate/up + GELU, down + gated
//   residual; then the final modulated norm + velocity projection + Euler update,
// separated by grid-wide barriers. Launch ramps and kernel-boundary cache maintenance are
// paid once per chunk instead of once per GEMM, and the weights of the next phase (and the
// prefix K/V tiles of the next attention) are already in flight while a barrier waits.
//
// Cross-workgroup coherence on gfx950 (8 XCDs, each with its own L2):
//  - every value produced in one phase and consumed in another by a different workgroup is
//    written with sc1 (device-scope, written through to memory) and the writer waits for
//    its stores before arriving at the barrier;
//  - values read by many workgroups (GEMM A operands, q, suffix K/V, norm statistics) live
//    in per-(step, layer) buffers that are written once per launch and never read before
//    that, aligned to 4 KB, so ordinary loads cannot hit a stale L2 line and each XCD's L2
//    serves the copies its CUs share;
//  - values rewritten every phase by their owner (the fp32 residual h, x, split partials)
//    are read with sc1 loads, which bypass the non-coherent L2.
// Every global access goes through a buffer descriptor whose extent is the allocation, so
// an index past a buffer reads zeros / drops the store instead of faulting. Every wait is
// bounded: a barrier that does not complete within ~2^20 polls records an error and lets
// every workgroup run to the end.
#include "fm_common.h"
#include "fm_kernels.h"
#include "fm_persist.h"

namespace fm {

constexpr int kPT = 512;                      // threads per workgroup: eight waves
constexpr int kPW = 8;
constexpr int kPCh = 4;                       // 32-wide k-chunks per wave and GEMM item
constexpr int kPKS = kPW * kPCh * 32;         // K covered by one GEMM item (1024)
constexpr int kLdr = 16;                      // LDS row stride (floats) of the wave partial tiles
constexpr uint32_t kSpinMax = 1u << 20;
constexpr uint32_t kAbort = 0xffffffffu;
constexpr int kCpSc1 = 16;                    // cache policy operand: sc1
constexpr int kMaxDa = 32;                    // action dims the in-projection unrolls over
constexpr uint32_t kOob = 0x80000000u;        // byte offset past every extent here (all < 2^31)

// ---------------------------------------------------------------------------------------
// Memory helpers
// ---------------------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int POL> __device__ __forceinline__ V16 ld16(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL); }
template <int POL> __device__ __forceinline__ u32x2 ld8(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL); }
template <int POL> __device__ __forceinline__ uint32_t ld4(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL); }
__device__ __forceinline__ void st16(Rsrc r, uint32_t off, V16 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpSc1); }
__device__ __forceinline__ void st8(Rsrc r, uint32_t off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpSc1); }
__device__ __forceinline__ void st4(Rsrc r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kCpSc1); }
__device__ __forceinline__ void st2(Rsrc r, uint32_t off, uint16_t v) { __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kCpSc1); }
__device__ __forceinline__ f32x4 as_f4(V16 v) { return __builtin_bit_cast(f32x4, v); }
__device__ __forceinline__ V16 as_v(f32x4 v) { return __builtin_bit_cast(V16, v); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) { return bf16_bits_rne(a) | (bf16_bits_rne(b) << 16); }

// Flag words: polled with volatile sc1 loads (never hoisted out of a wait loop).
__device__ __forceinline__ uint32_t flag_ld(const uint32_t* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ void flag_st(uint32_t* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 flag_ld4(const uint32_t* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
// all of this thread's memory operations (stores included) have completed
__device__ __forceinline__ void wait_all() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------------------
// Grid barrier: each workgroup publishes epoch e in its own flag word; workgroup 0 polls
// all of them with one 16-byte load per lane and then publishes e in the release word,
// which every workgroup polls. The caller's stores are complete before its flag is set.
// ---------------------------------------------------------------------------------------
// Waves 0-3 (store waves) do every global store of a phase and wait for all of their memory
// operations here; waves 4-7 (copy waves) also issue the buffer->LDS copies of the next
// phase's weights / key tiles, which stay in flight across the barrier and are waited for
// only before the barrier's final __syncthreads.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ bool copy_wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= 4; }

__device__ __forceinline__ void grid_sync(uint32_t* flags, uint32_t e) {
  const int tid = threadIdx.x;
  if (!copy_wave()) wait_all();
  __syncthreads();
  if (tid == 0) flag_st(flags + blockIdx.x, e);
  if (blockIdx.x == 0 && tid < 64) {
    const int G = gridDim.x;
    uint32_t n = 0, rel = e;
    while (true) {
      const u32x4 f = flag_ld4(flags + 4 * tid);
      bool ok = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) ok = ok && (4 * tid + j >= G || f[j] >= e);
      if (__all(ok)) break;
      if (++n > kSpinMax) { rel = kAbort; break; }
    }
    if (tid == 0) {
      if (rel == kAbort) flag_st(flags + kFlagErr, 1u);
      flag_st(flags + kFlagRelease, rel);
    }
  }
  if (tid == 0) {
    uint32_t n = 0;
    while (flag_ld(flags + kFlagRelease) < e) {
      if (++n > kSpinMax) { flag_st(flags + kFlagErr, 2u); break; }
    }
  }
  if (copy_wave()) wait_vm();
  __syncthreads();
}

// XCD-local flags: L2 atomics (executed in the XCD's L2, which its CUs share coherently).
__device__ __forceinline__ uint32_t l2_read(uint32_t* p) {
  uint32_t v;
  asm volatile("global_atomic_or %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p), "v"(0u) : "memory");
  return v;
}
__device__ __forceinline__ void l2_set(uint32_t* p, uint32_t v) {
  __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait (thread 0) until flags[i] >= e for i in [i0, i1).
__device__ __forceinline__ void wait_flags(uint32_t* flags, int i0, int i1, uint32_t e) {
  if (threadIdx.x == 0) {
    for (int i = i0; i < i1; ++i) {
      uint32_t n = 0;
      while (flag_ld(flags + i) < e) {
        if (++n > kSpinMax) { flag_st(flags + kFlagErr, 3u); break; }
      }
    }
  }
  __syncthreads();
}

// The loop description is read through the constant address space: it is never written
// while the kernel runs, so its fields load with scalar loads into SGPRs (uniform values,
// buffer descriptors as SGPR operands) instead of vector loads each waited on.
typedef const __attribute__((address_space(4))) LoopArgs LA;
typedef const __attribute__((address_space(4))) LayerW CLayerW;

// ---------------------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------------------
struct Smem {
  union {
    float red[2][kPW][64 * kLdr];             // wave partial tiles of up to two GEMM items
    V16 att[2][32 * 64];                      // two K / V^T key tiles (32 KB each)
  };
  V16 wbuf[2][kPW][kPCh][64];                 // next phase's weight fragments, per wave
  float2 ml[4][64];                           // attention wave-pair merge: (m, l)
  float aw[64][kMaxSA];                       // attention split weights per row of the tile
  float rinv[64];
};

// ---------------------------------------------------------------------------------------
// GEMM phase: items of 16 output columns x up to kPKS of K; a workgroup holds up to two
// items that share one K range (then nks == 1). Every load a phase needs (operands, norm
// statistics, epilogue vectors, residual) is issued before the first one is waited on, and
// the next phase's weights after them, so a phase costs one memory round trip.
// ---------------------------------------------------------------------------------------
struct GemmIn {
  const void* W; uint32_t wbytes;
  int N, K, nks, ntiles;
  const void* A; uint32_t lda, abytes;        // A [M x lda] bf16
  int xbase;                                  // split-K: first partial / flag slot of this GEMM
  bool w8;                                    // W holds FP8 codes (16 rows x 64 k per 1 KB fragment)
};

// Work item in slot s (0, 1) of this workgroup. Without split-K, items are column tiles
// dealt round-robin (two per workgroup at most). With split-K (one item per workgroup), the
// K splits of column tile n run on XCD n % 8 (workgroup b runs on XCD b % 8), in slots
// (n / 8) * nks + ks, so their partial tiles are exchanged through that XCD's L2.
struct GItem { int tile, ks, valid; };
__device__ __forceinline__ GItem gemm_item(const GemmIn& g, int s) {
  GItem it;
  if (g.nks == 1) {
    it.tile = (int)blockIdx.x + s * (int)gridDim.x;
    it.ks = 0;
  } else {
    const int x = blockIdx.x % 8, j = blockIdx.x / 8;
    it.tile = s == 0 ? (j / g.nks) * 8 + x : g.ntiles;
    it.ks = j % g.nks;
  }
  it.valid = it.tile < g.ntiles;
  if (!it.valid) { it.tile = 0; it.ks = 0; }
  return it;
}
__device__ __forceinline__ int gemm_slots(const GemmIn& g) {
  return gemm_item(g, 0).valid ? (gemm_item(g, 1).valid ? 2 : 1) : 0;
}

// Copy this workgroup's weight fragments of a phase (16 B per lane per k-chunk) into
// wbuf: each wave its own chunks, so a wave only waits for its own reads before reusing
// its part of the buffer. Absent fragments are zeros.
// Issued by the copy waves only (each serves its own section and that of wave w - 4), after
// every wave has read its current weights from wbuf (a __syncthreads after those reads).
__device__ __forceinline__ void prefetch_w(const GemmIn& g, Smem& sm) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4) return;
  V16 dw = make_desc(g.W, g.wbytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) dw[i] = __builtin_amdgcn_readfirstlane(dw[i]);   // uniform: SGPR operand
  const int kct = g.K / 32;
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int ws = wave - 4 + 4 * sec;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const GItem gi = gemm_item(g, s);
      const bool ok = gi.valid;
      const int tile = gi.tile, ks = gi.ks;
#pragma unroll
      for (int j = 0; j < kPCh; ++j) {
        const int c = ks * (kPKS / 32) + ws * kPCh + j;
        if (g.w8) {   // one 16-byte copy carries the FP8 codes of chunks c, c + 1 (j even)
          if (j & 1) continue;
          const uint32_t off = (ok && c < kct) ? (uint32_t)(((tile * (kct / 2) + c / 2) * 64 + lane) * 16) : kOob;
          dma16_lds(dw, lds_addr(&sm.wbuf[s][ws][j / 2][0]), off);
          continue;
        }
        const uint32_t off = (ok && c < kct) ? (uint32_t)(((tile * kct + c) * 64 + lane) * 16) : kOob;
        dma16_lds(dw, lds_addr(&sm.wbuf[s][ws][j][0]), off);
      }
    }
  }
}
// This wave's weight fragments from wbuf (the copies completed at the last barrier).
// Eight FP8 codes (two words, k order) to the bf16 MFMA operand, exactly (unscaled: the row
// scale is applied in the epilogue).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ V16 fp8x8_bf16(uint32_t w0, uint32_t w1) {
  return V16{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
}
__device__ __forceinline__ void read_w(const Smem& sm, V16 (&wr)[2][kPCh], int nslot, bool w8) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (w8) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < kPCh; j += 2) {
        const V16 x = s < nslot ? sm.wbuf[s][wave][j / 2][lane] : vzero();
        wr[s][j] = fp8x8_bf16(x[0], x[1]);
        wr[s][j + 1] = fp8x8_bf16(x[2], x[3]);
      }
    return;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < kPCh; ++j) wr[s][j] = s < nslot ? sm.wbuf[s][wave][j][lane] : vzero();
}

// A fragments of this workgroup's K range: lane l holds row 16 mb + l % 16, k run l / 16.
// Activation operands (the GEMM A inputs hs, attention output, GELU.up output) are stored
// fragment-major: 16 x 32 blocks (row block r / 16, k-chunk k / 32) of 1 KB, row-block
// major, lane (r % 16) + 16 ((k % 32) / 8) holding 8 consecutive k. A fragment load is then
// one contiguous kilobyte (8 whole cache lines) instead of 16 rows x 64 bytes. Byte offset
// of element (r, k) of a K-wide operand:
__device__ __forceinline__ uint32_t act_off(int r, int k, int K) {
  return (uint32_t)(((((r >> 4) * (K >> 5) + (k >> 5)) * 64 + (r & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7)) * 2);
}
// Folded attention row of query head n, token i of request b: requests hold nq H rows
// (head-major), padded to whole 16-row blocks.
__device__ __forceinline__ int q_row(LA& a, int b, int n, int i) {
  return b * ((a.nq * a.H + 15) & ~15) + n * a.H + i;
}
// bytes of a K-wide operand of M rows (whole row blocks)
__device__ __forceinline__ uint32_t act_bytes(int M, int K) { return (uint32_t)(((M + 15) & ~15) * K * 2); }

__device__ __forceinline__ void load_a(const GemmIn& g, int M, V16 (&ra)[kPCh][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Rsrc rA = make_rsrc(g.A, g.abytes);
  const int kct = g.K / 32;
  const int ks = gemm_item(g, 0).ks;
#pragma unroll
  for (int j = 0; j < kPCh; ++j) {
    const int c = ks * (kPKS / 32) + wave * kPCh + j;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int row = 16 * mb + (lane & 15);
      ra[j][mb] = ld16<0>(rA, (row < M && c < kct) ? (uint32_t)(((mb * kct + c) * 64 + lane) * 16) : kOob);
    }
  }
}

// Per-row 1 / RMS of a norm input from the producer's partial sums of squares (stats
// [M][D / 16], D a multiple of 512 and at most 2048): thread t covers a quarter... an eighth
// of row t / 8, up to four 16-byte loads.
struct StatLoad {
  V16 v[4];
  __device__ __forceinline__ void issue(const void* stats, int M, int D) {
    const int t = threadIdx.x, r = t >> 3, part = t & 7;
    const int nt = D / 16, per = nt / 8;
    const Rsrc rs = make_rsrc(stats, (uint32_t)(M * nt * 4));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = ld16<0>(rs, (r < M && 4 * j < per) ? (uint32_t)((r * nt + part * per + 4 * j) * 4) : kOob);
  }
  __device__ __forceinline__ void finish(int D, float eps, Smem& sm) const {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 f = as_f4(v[j]);
      s += (f[0] + f[1]) + (f[2] + f[3]);
    }
    s = group_sum<8>(s);
    if ((threadIdx.x & 7) == 0) sm.rinv[threadIdx.x >> 3] = rsqrtf(s / (float)D + eps);
  }
};

// 16 bytes of a per-column fp32 vector at column n (vectors padded to 4 floats); zeros
// without a memory access where ok is false (threads that do not use the value)
__device__ __forceinline__ V16 col4(const float* p, int n, int limit, bool ok = true) {
  const Rsrc r = make_rsrc(p, (uint32_t)(limit * 4));
  return ld16<0>(r, ok ? (uint32_t)(n * 4) : kOob);
}

// MFMA over the workgroup's K range, then the wave partials summed in LDS: thread t < 256
// gets, in v[s], the 4-column run (row t / 4, columns 4 (t % 4)) of item slot s.
__device__ __forceinline__ void gemm_core(const V16 (&wr)[2][kPCh], const V16 (&ra)[kPCh][4], Smem& sm, int nslot,
                                          f32x4 (&v)[2]) {
  typedef Mma<bf16> MT;
  typedef MT::frag frag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 acc[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[s][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kPCh; ++j)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      acc[0][mb] = MT::mma(__builtin_bit_cast(frag, ra[j][mb]), __builtin_bit_cast(frag, wr[0][j]), acc[0][mb]);
      if (nslot > 1) acc[1][mb] = MT::mma(__builtin_bit_cast(frag, ra[j][mb]), __builtin_bit_cast(frag, wr[1][j]), acc[1][mb]);
    }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (s >= nslot) break;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.red[s][wave][(16 * mb + 4 * (lane >> 4) + e) * kLdr + (lane & 15)] = acc[s][mb][e];
  }
  __syncthreads();
  const int t = threadIdx.x, r = (t & 255) >> 2, q = t & 3;
  v[0] = v[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (t < 256) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s >= nslot) break;
#pragma unroll
      for (int w = 0; w < kPW; ++w) v[s] += *(const f32x4*)&sm.red[s][w][r * kLdr + 4 * q];
    }
  }
}

// Split-K: items with ks > 0 publish their partial tile and flag; the ks == 0 item waits for
// the others and adds them in ks order. Returns false for the publishing items.
__device__ __forceinline__ bool split_reduce(LA& a, const GemmIn& g, uint32_t e, f32x4& v) {
  if (g.nks == 1) return true;
  const GItem gi = gemm_item(g, 0);
  const int idx = g.xbase + gi.tile * g.nks;   // slot of split 0 of this tile
  const int t = threadIdx.x, lane = t & 63, r = (t & 255) >> 2, q = t & 3;
  // partials: ordinary stores into this XCD's L2, read by the tile's owner on the same XCD
  const Rsrc rp = make_rsrc(a.ws_split, (uint32_t)(kMaxSplitItems * 64 * 16 * 4));
  uint32_t* fl = a.flags + kFlagSplit + idx;
  if (gi.ks > 0) {
    if (t < 256 && r < a.M)
      __builtin_amdgcn_raw_buffer_store_b128(as_v(v), rp, (uint32_t)((((idx + gi.ks) * 64 + r) * 16 + 4 * q) * 4), 0, 0);
    if (!copy_wave()) wait_all();   // the copy waves' loads may stay in flight
    __syncthreads();
    if (t == 0) l2_set(fl + gi.ks, e);
    return false;
  }
  if (t < 64) {
    uint32_t n = 0;
    while (true) {
      const uint32_t f = (lane >= 1 && lane < g.nks) ? l2_read(fl + lane) : 0xffffffffu;
      if (__all(f >= e)) break;
      if (++n > kSpinMax) { if (lane == 0) flag_st(a.flags + kFlagErr, 3u); break; }
    }
  }
  __syncthreads();
  if (t < 256 && r < a.M) {
    asm volatile("buffer_inv sc0" ::: "memory");   // no stale partial line in this CU's L1
    V16 p[3];
#pragma unroll
    for (int k = 1; k < 4; ++k) p[k - 1] = ld16<0>(rp, k < g.nks ? (uint32_t)((((idx + k) * 64 + r) * 16 + 4 * q) * 4) : kOob);
#pragma unroll
    for (int k = 1; k < 4; ++k) v += as_f4(p[k - 1]);
  }
  return true;
}

// Residual epilogue inputs of thread (row r, columns n..n+3): gate, next scale, h (sc1).
struct ResidIn {
  V16 g, sc, h, ws;   // ws: FP8 row scales of the weight (ones for bf16 weights)
  __device__ __forceinline__ void issue(LA& a, int r, int n, const float* gate, const float* scale_next, bool use,
                                        const float* wscale) {
    g = col4(gate, n, a.D, use);
    sc = col4(scale_next, n, a.D, use);
    ws = wscale ? col4(wscale, n, a.D, use) : as_v(f32x4{1.f, 1.f, 1.f, 1.f});
    const Rsrc rh = make_rsrc(a.h, (uint32_t)(a.M * a.D * 4));
    h = ld16<kCpSc1>(rh, (use && r < a.M) ? (uint32_t)((r * a.D + n) * 4) : kOob);
  }
};

// h += gate * y; hs = bf16(h (1 + scale of the next norm)); partial sum of squares of h
// over the item's 16 columns (four consecutive lanes hold one row's 16 columns)
__device__ __forceinline__ void epi_resid(LA& a, f32x4 v, const ResidIn& in, int r, int n, int tile,
                                          char* hs_out, float* st_out) {
  const bool ok = r < a.M;
  const f32x4 hv = as_f4(in.h) + as_f4(in.g) * (as_f4(in.ws) * v);
  const f32x4 sc = as_f4(in.sc);
  float ss = hv[0] * hv[0] + hv[1] * hv[1] + hv[2] * hv[2] + hv[3] * hv[3];
  ss = group_sum<4>(ss);
  if (ok) {
    const Rsrc rh = make_rsrc(a.h, (uint32_t)(a.M * a.D * 4));
    st16(rh, (uint32_t)((r * a.D + n) * 4), as_v(hv));
    const Rsrc rs = make_rsrc(hs_out, act_bytes(a.M, a.D));
    st8(rs, act_off(r, n, a.D),
        u32x2{pack_bf2(hv[0] * (1.f + sc[0]), hv[1] * (1.f + sc[1])), pack_bf2(hv[2] * (1.f + sc[2]), hv[3] * (1.f + sc[3]))});
    if ((threadIdx.x & 3) == 0) {
      const Rsrc rt = make_rsrc(st_out, (uint32_t)(a.M * (a.D / 16) * 4));
      st4(rt, (uint32_t)((r * (a.D / 16) + tile) * 4), __float_as_uint(ss));
    }
  }
}

// ---------------------------------------------------------------------------------------
// Attention (heads folded into rows; transposed S^T = K Q^T, O^T = V^T P^T as in the
// stand-alone attention kernel). One item = 64 query rows of one request x a split of up to
// two 32-key tiles; waves w and w + 4 share query rows and take one tile each, then merge.
// Key tiles are listed prefix first (pool, ceil(P / 32) tiles), then suffix (this step's
// own K/V, ceil(H / 32) tiles).
// ---------------------------------------------------------------------------------------
constexpr int kDH = 256;
constexpr int kDB = kDH / 16, kDCH = kDH / 32;
constexpr int kFK = 2 * kDCH, kFV = kDB;        // K and V^T fragments of one tile
constexpr int kFT = kFK + kFV;
constexpr int kFPW = kFT / kPW;                 // fragments per wave per tile
static_assert(kFT % kPW == 0, "tile fragments per wave");

struct AttnItem { int valid, b, rt, sp, pb; };   // pb: the request's compact prefix length

// All key splits of one row tile run on one XCD (workgroup b runs on XCD b % 8): their
// partial results stay in that XCD's L2, which every CU of the XCD sees coherently, and
// the splits synchronize among themselves through L2 atomics. Row tile rb of the B * RT
// goes to XCD rb % 8, split sp to slot (rb / 8) * SA + sp of that XCD.
// pb: the item's compact prefix length (attn_item_pb, loaded once per launch)
__device__ __forceinline__ AttnItem attn_item(LA& a, int pb) {
  AttnItem it;
  const int x = blockIdx.x % 8, j = blockIdx.x / 8;
  const int rb = (j / a.SA) * 8 + x;
  it.sp = j % a.SA;
  it.b = rb / a.RT;
  it.rt = rb % a.RT;
  it.valid = rb < a.B * a.RT;
  it.pb = pb;
  return it;
}
__device__ __forceinline__ int attn_item_pb(LA& a) {
  const AttnItem it = attn_item(a, 0);
  typedef const __attribute__((address_space(4))) int CI;
  return it.valid ? *(CI*)(a.plens + __builtin_amdgcn_readfirstlane(it.b)) : 0;
}

// Key tile `which` (0/1) of split sp: tiles sp and sp + SA, so that this step's suffix tiles
// (the last ones, written by the QKV phase just before and loaded only after its barrier)
// fall to different splits instead of doubling one split's loads.
__device__ __forceinline__ int attn_tile(LA& a, const AttnItem& it, int which) { return it.sp + which * a.SA; }

// Issue the copies of key tile `which` (0/1) of the item into LDS: prefix tiles only when
// suffix == false, suffix tiles only when suffix == true.
__device__ __forceinline__ void attn_issue(LA& a, const AttnItem& it, int l, const char* rot_l, int which,
                                           bool suffix, Smem& sm) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // prefix tiles: the copy waves, each its own and wave w - 4's fragments; suffix tiles:
  // every wave its own
  if (!suffix && wave < 4) return;
  const int ti = attn_tile(a, it, which);
  if (!it.valid || ti >= a.TP + a.TS) return;
  const bool is_suf = ti >= a.TP;
  if (is_suf != suffix) return;
  if (!is_suf && 32 * ti >= it.pb) return;   // past the request's own prefix: nothing it sees
  V16 dk, dv;
  int kt, vds;
  if (!is_suf) {
    const bf16* kp = a.pool + (size_t)(2 * l) * a.plane + (size_t)it.b * a.cap * kDH;
    const bf16* vp = a.pool + (size_t)(2 * l + 1) * a.plane + (size_t)it.b * kDH * a.cap;
    dk = make_desc(kp, (uint32_t)(a.cap * kDH * 2));
    dv = make_desc(vp, (uint32_t)(kDH * a.cap * 2));
    kt = 32 * ti; vds = a.cap;
  } else {
    const char* sk = rot_l + a.o_sk + (size_t)it.b * a.Hp * kDH * 2;
    const char* sv = rot_l + a.o_svt + (size_t)it.b * kDH * a.Hp * 2;
    dk = make_desc(sk, (uint32_t)(a.Hp * kDH * 2));
    dv = make_desc(sv, (uint32_t)(kDH * a.Hp * 2));
    kt = 32 * (ti - a.TP); vds = a.Hp;
  }
  const uint32_t lds0 = lds_addr(&sm.att[which][0]);
  const int nsec = suffix ? 1 : 2;
  for (int sec = 0; sec < nsec; ++sec)
#pragma unroll
  for (int i = 0; i < kFPW; ++i) {
    const int f = (suffix ? wave : wave - 4 + 4 * sec) * kFPW + i;
    uint32_t off;
    if (is_suf) {   // this step's K and V^T are fragment-major: contiguous kilobytes
      if (f < kFK) {
        const int kb = f / kDCH, c = f % kDCH;
        off = (uint32_t)(((((kt >> 4) + kb) * kDCH + c) * 64 + lane) * 16);
      } else {
        const int db = f - kFK;
        off = (uint32_t)(((db * (vds >> 5) + (kt >> 5)) * 64 + lane) * 16);
      }
    } else if (f < kFK) {
      const int kb = f / kDCH, c = f % kDCH;
      off = (uint32_t)(((kt + 16 * kb + (lane & 15)) * kDH + c * 32 + (lane >> 4) * 8) * 2);
    } else {
      const int db = f - kFK;
      off = (uint32_t)(((16 * db + (lane & 15)) * vds + kt + (lane >> 4) * 8) * 2);
    }
    V16 d = f < kFK ? dk : dv;
#pragma unroll
    for (int u = 0; u < 4; ++u) d[u] = __builtin_amdgcn_readfirstlane(d[u]);   // uniform: SGPR operand
    dma16_lds(d, lds0 + (uint32_t)f * 1024u, off);
  }
}

__device__ __forceinline__ void attn_phase(LA& a, int pb, int l, const char* rot_l, Smem& sm, uint32_t e_attn,
                                           const GemmIn& gin_o_next) {
  typedef Mma<bf16> MT;
  typedef MT::frag frag;
  const AttnItem it = attn_item(a, pb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w4 = wave & 3, half = wave >> 2;
  frag qf[kDCH];
  {
    // q is stored fragment-major over the folded rows of each request (q_row): the 16 rows
    // of this wave are one contiguous kilobyte per 32-wide d chunk
    const int R = a.nq * a.H, Rp = (R + 15) & ~15;
    const int rloc = it.rt * 64 + 16 * w4 + (lane & 15);
    const int blk = (it.b * Rp + it.rt * 64 + 16 * w4) >> 4;
    const Rsrc rq = make_rsrc(rot_l + a.o_q, (uint32_t)(a.B * Rp * kDH * 2));
#pragma unroll
    for (int c = 0; c < kDCH; ++c)
      qf[c] = __builtin_bit_cast(frag, ld16<0>(rq, (it.valid && rloc < R) ? (uint32_t)(((blk * kDCH + c) * 64 + lane) * 16) : kOob));
  }
  // the suffix tiles are this phase's inputs: copy them now (prefix tiles were issued
  // before the barrier)
  attn_issue(a, it, l, rot_l, 0, true, sm);
  attn_issue(a, it, l, rot_l, 1, true, sm);
  wait_all();
  __syncthreads();

  const int ti = attn_tile(a, it, half);
  // a tile with a key the request sees: a suffix tile, or a prefix tile that starts inside
  // the request's compact prefix
  const bool has = it.valid && ti < a.TP + a.TS && (ti >= a.TP || 32 * ti < it.pb);
  f32x4 o[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // a half without such a tile keeps (O, l) = 0 and a finite reference below any score, which
  // the merges below weigh by exp2(-1e30 - m) = 0
  float m = -1e30f, lsum = 0.f;
  if (has) {
    const V16* sK = &sm.att[half][0];
    const V16* sV = sK + kFK * 64;
    const bool is_suf = ti >= a.TP;
    const int kbase = is_suf ? 32 * (ti - a.TP) : 32 * ti;
    const int klim = is_suf ? a.H : it.pb;
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      V16 kf[kDCH];
#pragma unroll
      for (int c = 0; c < kDCH; ++c) kf[c] = sK[(kb * kDCH + c) * 64 + lane];
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
      for (int c = 0; c < kDCH; c += 2) {
        s0 = MT::mma(__builtin_bit_cast(frag, kf[c]), qf[c], s0);
        s1 = MT::mma(__builtin_bit_cast(frag, kf[c + 1]), qf[c + 1], s1);
      }
      s[kb] = s0 + s1;
    }
    const int kl = kbase + 4 * (lane >> 4);
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = (kl + 16 * kb + e < klim) ? s[kb][e] * a.scale_log2 : -INFINITY;
        s[kb][e] = v;
        mt = fmaxf(mt, v);
      }
    m = group4_max(mt);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = exp2f(s[kb][e] - m);
        s[kb][e] = p;
        ls += p;
      }
    lsum = group4_sum(ls);
    const frag pf = frag{(bf16)s[0][0], (bf16)s[0][1], (bf16)s[0][2], (bf16)s[0][3],
                         (bf16)s[1][0], (bf16)s[1][1], (bf16)s[1][2], (bf16)s[1][3]};
#pragma unroll
    for (int db = 0; db < kDB; ++db) o[db] = MT::mma(__builtin_bit_cast(frag, sV[db * 64 + lane]), pf, o[db]);
  }
  __syncthreads();   // every wave has read its tile: the tile buffers hold the merge now
  f32x4* mrg = (f32x4*)&sm.att[0][0];   // [w4][db][lane]
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db) mrg[(w4 * kDB + db) * 64 + lane] = o[db];
    sm.ml[w4][lane] = make_float2(m, lsum);
  }
  __syncthreads();
  const int rb = it.b * a.RT + it.rt;
  const int item = rb * a.SA + it.sp;
  // this split's partial (unnormalized O, m, l), in the MFMA output layout; ordinary stores:
  // it is read only by the other splits of the row tile, all on this XCD
  const Rsrc rw = make_rsrc(a.ws_attn, (uint32_t)(kMaxAttnItems * 64 * kDH * 4));
  const Rsrc rm = make_rsrc(a.ws_attn_ml, (uint32_t)(kMaxAttnItems * 64 * 8));
  if (half == 0 && it.valid) {
    const float2 p2 = sm.ml[w4][lane];
    const float mx = fmaxf(m, p2.x);
    const float a1 = exp2f(m - mx), a2 = exp2f(p2.x - mx);
    const uint32_t ob = (uint32_t)(item * 64 * kDH * 4);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const f32x4 v = a1 * o[db] + a2 * mrg[(w4 * kDB + db) * 64 + lane];
      __builtin_amdgcn_raw_buffer_store_b128(as_v(v), rw, ob + (uint32_t)(((w4 * kDB + db) * 64 + lane) * 16), 0, 0);
    }
    if (lane < 16) {
      const float2 ml = make_float2(mx, a1 * lsum + a2 * p2.y);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(ml.x), __float_as_uint(ml.y)}, rm,
                                            (uint32_t)((item * 64 + 16 * w4 + lane) * 8), 0, 0);
    }
  }
  // the splits of the row tile meet: publish this one, wait for all of them
  if (!copy_wave()) wait_all();
  __syncthreads();
  // O projection weights for the next phase (copy waves; no load of theirs follows): issued
  // before the wait for the other splits, so they arrive during it instead of competing
  // with the merge's loads
  prefetch_w(gin_o_next, sm);
  uint32_t* fl = a.flags + kFlagAttn + rb * kMaxSA;
  if (threadIdx.x == 0 && it.valid) l2_set(fl + it.sp, e_attn);
  if (threadIdx.x < 64 && it.valid) {
    uint32_t n = 0;
    while (true) {
      const uint32_t f = lane < a.SA ? l2_read(fl + lane) : 0xffffffffu;
      if (__all(f >= e_attn)) break;
      if (++n > kSpinMax) { if (lane == 0) flag_st(a.flags + kFlagErr, 5u); break; }
    }
  }
  __syncthreads();
  const int SA = a.SA;
  const bool merger = it.valid && threadIdx.x < 256;
  // per row of the tile, the split weights exp2(m_s - max) / sum_s exp2(m_s - max) l_s:
  // thread (row t / 4, quarter t % 4) reads splits q, q + 4, q + 8, q + 12
  if (merger) {
    asm volatile("buffer_inv sc0" ::: "memory");   // this CU's L1 holds no stale partial line
    const int rl = threadIdx.x >> 2, q = threadIdx.x & 3;
    u32x2 mlv[kMaxSA / 4];
#pragma unroll
    for (int u = 0; u < kMaxSA / 4; ++u) {
      const int sp = q + 4 * u;
      mlv[u] = __builtin_amdgcn_raw_buffer_load_b64(rm, sp < SA ? (uint32_t)(((rb * SA + sp) * 64 + rl) * 8) : kOob, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kMaxSA / 4; ++u)
      if (q + 4 * u < SA) mx = fmaxf(mx, __uint_as_float(mlv[u][0]));
    mx = fmaxf(mx, dpp_mov<kDppXor1>(mx));
    mx = fmaxf(mx, dpp_mov<kDppXor2>(mx));
    float wv[kMaxSA / 4], den = 0.f;
#pragma unroll
    for (int u = 0; u < kMaxSA / 4; ++u) {
      wv[u] = q + 4 * u < SA ? exp2f(__uint_as_float(mlv[u][0]) - mx) : 0.f;
      den += wv[u] * __uint_as_float(mlv[u][1]);
    }
    den = group_sum<4>(den);
    const float inv = 1.f / den;
#pragma unroll
    for (int u = 0; u < kMaxSA / 4; ++u) sm.aw[rl][q + 4 * u] = wv[u] * inv;
  }
  __syncthreads();
  if (!it.valid) return;
  // merge this split's share of the row tile: thread = 4 consecutive head dims of one row,
  // every wave taking items (all of an item's loads issued together)
  constexpr int PER_TILE = 64 * kDH / 4;
  const int per = (PER_TILE + SA - 1) / SA;
  const int beg = it.sp * per, end = min(PER_TILE, beg + per);
  const Rsrc rao = make_rsrc(rot_l + a.o_ao, act_bytes(a.M, a.qd));
  const int R = a.nq * a.H;
  if (copy_wave()) asm volatile("buffer_inv sc0" ::: "memory");   // as the mergers above
  for (int w0 = beg + (int)threadIdx.x; w0 < end; w0 += 512) {
    V16 ov[1][kMaxSA];
#pragma unroll
    for (int sp = 0; sp < kMaxSA; ++sp)
      ov[0][sp] = ld16<0>(rw, sp < SA ? (uint32_t)(((rb * SA + sp) * 64 * kDH + w0 * 4) * 4) : kOob);
    __builtin_amdgcn_sched_barrier(0);   // every load in flight before the first use
#pragma unroll
    for (int h2 = 0; h2 < 1; ++h2) {
      const int w = w0;
      const int ln = w & 63, db = (w >> 6) % kDB, ww = w / (64 * kDB);
      const int rl = 16 * ww + (ln & 15);
      f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < kMaxSA; ++sp)
        if (sp < SA) num += sm.aw[rl][sp] * as_f4(ov[h2][sp]);
      const int r = it.rt * 64 + rl;
      if (r < R) {
        const int n = r / a.H, t = r % a.H;
        const uint32_t off = act_off(it.b * a.H + t, n * kDH + db * 16 + 4 * (ln >> 4), a.qd);
        st8(rao, off, u32x2{pack_bf2(num[0], num[1]), pack_bf2(num[2], num[3])});
      }
    }
  }
  // the copy waves stored merge results too: they complete before this workgroup arrives at
  // the barrier (grid_sync waits only for the store waves' memory operations); their O
  // weight copies, issued before the wait for the splits, are waited for with them
  if (copy_wave()) wait_all();
}

// ---------------------------------------------------------------------------------------
// The loop kernel
// ---------------------------------------------------------------------------------------
// The kernel's arguments are re-read through an opaque pointer at every step and layer
// (launder): values derived from them are then recomputed where used instead of being
// hoisted out of the loops and held in registers (or spilled) across every phase.
__device__ __forceinline__ LA& launder(const LoopArgs* p) {
  LA* q = (LA*)p;
  asm volatile("" : "+s"(q));
  return *q;
}
__device__ __forceinline__ LayerW layer_w(LA& a, int l) {
  CLayerW* p = (CLayerW*)a.lw + l;
  return LayerW{p->qkv, p->o, p->gu, p->down, p->sqkv, p->so, p->sgu, p->sdown};
}

// W8: the per-layer weights are FP8 codes with per-row scales (see read_w)
template <bool W8>
__global__ void __launch_bounds__(kPT, 1) k_loop(const LoopArgs* __restrict__ pa, LaunchArgs la) {
  __shared__ Smem sm;
  const int t = threadIdx.x, G = gridDim.x;
  uint32_t e = la.e0;
  // epilogue thread coordinates: item slot, row, 4-column run
  const int er = (t & 255) >> 2, eq = t & 3;

  auto rot = [&](LA& a, int kk, int l) -> char* { return a.rot + (size_t)kk * a.rot_step + (size_t)l * a.rot_layer; };
  auto gin_qkv = [&](LA& a, const void* W, char* rl) {
    const int D = a.D, M = a.M;
    GemmIn g;
    g.W = W; g.wbytes = a.wb_qkv; g.N = a.nqkv; g.K = D; g.nks = (D + kPKS - 1) / kPKS;
    g.ntiles = (a.nqkv + 15) / 16; g.A = rl + a.o_hs; g.lda = D; g.abytes = act_bytes(M, D); g.xbase = 0; g.w8 = W8;
    return g;
  };
  auto gin_o = [&](LA& a, const void* W, char* rl) {
    const int D = a.D, M = a.M;
    GemmIn g;
    g.W = W; g.wbytes = a.wb_o; g.N = D; g.K = a.qd; g.nks = (a.qd + kPKS - 1) / kPKS;
    g.ntiles = D / 16; g.A = rl + a.o_ao; g.lda = a.qd; g.abytes = act_bytes(M, a.qd); g.xbase = 0; g.w8 = W8;
    return g;
  };
  auto gin_up = [&](LA& a, const void* W, char* rl) {
    const int D = a.D, M = a.M;
    GemmIn g;
    g.W = W; g.wbytes = a.wb_gu; g.N = 2 * a.F; g.K = D; g.nks = (D + kPKS - 1) / kPKS;
    g.ntiles = 2 * a.F / 16; g.A = rl + a.o_hsu; g.lda = D; g.abytes = act_bytes(M, D); g.xbase = 0; g.w8 = W8;
    return g;
  };
  auto gin_down = [&](LA& a, const void* W, char* rl) {
    const int D = a.D, M = a.M;
    GemmIn g;
    g.W = W; g.wbytes = a.wb_down; g.N = D; g.K = a.F; g.nks = (a.F + kPKS - 1) / kPKS;
    g.ntiles = D / 16; g.A = rl + a.o_act; g.lda = a.F; g.abytes = act_bytes(M, a.F); g.xbase = kMaxSplitItems / 2; g.w8 = W8;
    return g;
  };
  auto gin_out = [&](LA& a, char* rf) {
    const int D = a.D, M = a.M;
    GemmIn g;
    g.W = a.w_out; g.wbytes = a.wb_out; g.N = a.da; g.K = D; g.nks = (D + kPKS - 1) / kPKS;
    g.ntiles = (a.da + 15) / 16; g.A = rf + a.o_hs; g.lda = D; g.abytes = act_bytes(M, D); g.xbase = 0; g.w8 = false;
    return g;
  };
  // the table row of site s at step k: [scale | shift | gate], D each
  auto site = [&](LA& a, int k, int s, int part) { return a.table + ((size_t)k * a.S + s) * 3 * a.D + (size_t)part * a.D; };
  auto cvec = [&](LA& a, int k, int s) {
    const long off = s == 2 * a.L ? (long)a.L * (a.cq4 + a.cg4) : (long)(s / 2) * (a.cq4 + a.cg4) + (s % 2) * a.cq4;
    return a.cbuf + (size_t)k * a.csum + off;
  };

  int pb;   // this workgroup's attention item: its request's compact prefix length
  {
    LA& a = launder(pa);
    prefetch_w(gin_qkv(a, layer_w(a, 0).qkv, rot(a, 0, 0)), sm);
    pb = attn_item_pb(a);
  }
  for (int kk = 0; kk < la.nsteps; ++kk) {
    LA& a = launder(pa);
    const int k = la.k0 + kk;
    const int D = a.D, M = a.M;
    const Rsrc rx = make_rsrc(a.x, (uint32_t)(M * a.da * 4));
    // ---- in-projection: h = x W_in^T + b_in; hs, statistics of norm site 0 ----------
    // (store waves: thread t = row t / 4, columns 4 (t % 4) .. + 3 of the 16-column tile)
    {
      char* r0 = rot(a, kk, 0);
      if ((int)blockIdx.x < D / 16 && t < 256) {
        const int r = t >> 2, n = (int)blockIdx.x * 16 + 4 * (t & 3);
        const bool ok = r < M;
        const Rsrc rw = make_rsrc(a.w_in, (uint32_t)(D * a.da * 2));
        V16 xv[kMaxDa / 4];
        u32x2 w[4][kMaxDa / 4];
#pragma unroll
        for (int j = 0; j < kMaxDa / 4; ++j) {
          const bool in = 4 * j < a.da;
          xv[j] = ld16<kCpSc1>(rx, (ok && in) ? (uint32_t)((r * a.da + 4 * j) * 4) : kOob);
#pragma unroll
          for (int c = 0; c < 4; ++c) w[c][j] = ld8<0>(rw, in ? (uint32_t)(((n + c) * a.da + 4 * j) * 2) : kOob);
        }
        const V16 bb = col4(a.b_in, n, D);
        const V16 sc = col4(site(a, k, 0, 0), n, D);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 h = as_f4(bb);
#pragma unroll
        for (int j = 0; j < kMaxDa / 4; ++j) {
          const f32x4 x4 = as_f4(xv[j]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float wf[4] = {__uint_as_float(w[c][j][0] << 16), __uint_as_float(w[c][j][0] & 0xffff0000u),
                                 __uint_as_float(w[c][j][1] << 16), __uint_as_float(w[c][j][1] & 0xffff0000u)};
#pragma unroll
            for (int u = 0; u < 4; ++u) h[c] += x4[u] * wf[u];
          }
        }
        const f32x4 s4 = as_f4(sc);
        const float ss = group_sum<4>(h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3]);
        if (ok) {
          const Rsrc rh = make_rsrc(a.h, (uint32_t)(M * D * 4));
          st16(rh, (uint32_t)((r * D + n) * 4), as_v(h));
          const Rsrc rs = make_rsrc(r0 + a.o_hs, act_bytes(M, D));
          st8(rs, act_off(r, n, D),
              u32x2{pack_bf2(h[0] * (1.f + s4[0]), h[1] * (1.f + s4[1])), pack_bf2(h[2] * (1.f + s4[2]), h[3] * (1.f + s4[3]))});
          if ((t & 3) == 0) {
            const Rsrc rt = make_rsrc(r0 + a.o_st, (uint32_t)(M * (D / 16) * 4));
            st4(rt, (uint32_t)((r * (D / 16) + (int)blockIdx.x) * 4), __float_as_uint(ss));
          }
        }
      }
      grid_sync(a.flags, ++e);
    }

    for (int l = 0; l < a.L; ++l) {
      LA& a = launder(pa);
      const int D = a.D, M = a.M;
      char* rl = rot(a, kk, l);
      const LayerW lw = layer_w(a, l);
      const AttnItem ait = attn_item(a, pb);
      // ---- QKV + RoPE: q to the q buffer, k / v to this step's suffix K / V^T ---------
      {
        const GemmIn g = gin_qkv(a, lw.qkv, rl);
        const int nslot = gemm_slots(g);
        V16 wr[2][kPCh];
        read_w(sm, wr, nslot, g.w8);
        V16 ra[kPCh][4];
        load_a(g, M, ra);
        StatLoad st;
        st.issue(rl + a.o_st, M, D);
        const int b = er / a.H, i = er % a.H;
        const Rsrc rc = make_rsrc(a.rope_cs, (uint32_t)(a.B * a.H * (kDH / 2) * 8));
        V16 cv[2], csv[2], wsv[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int n = ((int)blockIdx.x + s2 * G) * 16 + 4 * eq;
          const bool use = t < 256 && s2 < nslot && er < M;
          cv[s2] = col4(cvec(a, k, 2 * l), min(n, a.cq4 - 4), a.cq4, use);
          wsv[s2] = W8 ? col4(lw.sqkv, min(n, a.cq4 - 4), a.cq4, use) : as_v(f32x4{1.f, 1.f, 1.f, 1.f});
          csv[s2] = ld16<0>(rc, (use && a.rope && n < a.qd + kDH) ? (uint32_t)((er * (kDH / 2) + (n % kDH) / 2) * 8) : kOob);
        }
        st.finish(D, a.eps, sm);
        f32x4 v[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if (nslot) gemm_core(wr, ra, sm, nslot, v);
        __syncthreads();   // rinv visible; every read of the wave partial tiles is done
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int n = ((int)blockIdx.x + s2 * G) * 16 + 4 * eq;
          if (t < 256 && s2 < nslot && er < M && n < a.nqkv) {
            f32x4 y = sm.rinv[er] * (as_f4(wsv[s2]) * v[s2]) + as_f4(cv[s2]);
            if (a.rope && n < a.qd + kDH) {
              const f32x4 cs = as_f4(csv[s2]);
              const float x0 = y[0], x1 = y[1], x2 = y[2], x3 = y[3];
              y[0] = x0 * cs[0] - x1 * cs[1];
              y[1] = x1 * cs[0] + x0 * cs[1];
              y[2] = x2 * cs[2] - x3 * cs[3];
              y[3] = x3 * cs[2] + x2 * cs[3];
            }
            if (n < a.qd) {
              const int Rp = (a.nq * a.H + 15) & ~15;
              const Rsrc rq = make_rsrc(rl + a.o_q, (uint32_t)(a.B * Rp * kDH * 2));
              st8(rq, act_off(q_row(a, b, n / kDH, i), n % kDH, kDH), u32x2{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])});
            } else if (n < a.qd + kDH) {
              // this step's K ([b][Hp keys][dh]) and V^T ([b][dh][Hp key slots]) fragment-major
              const Rsrc rk = make_rsrc(rl + a.o_sk, (uint32_t)(a.B * a.Hp * kDH * 2));
              st8(rk, act_off(b * a.Hp + i, n - a.qd, kDH), u32x2{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])});
            } else {
              const Rsrc rv = make_rsrc(rl + a.o_svt, (uint32_t)(a.B * kDH * a.Hp * 2));
              const int d0 = n - a.qd - kDH;
              const int slot = vt_slot<bf16>(i);
#pragma unroll
              for (int j = 0; j < 4; ++j)
                st2(rv, act_off(b * kDH + d0 + j, slot, a.Hp), __builtin_bit_cast(uint16_t, (bf16)y[j]));
            }
          }
        }
        // prefix tiles of this layer's attention item, into the buffer the partial tiles
        // used; in flight across the barrier. Issued after the stores above, which the
        // barrier waits for and which would otherwise queue behind these copies.
        __syncthreads();
        attn_issue(a, ait, l, rl, 0, false, sm);
        attn_issue(a, ait, l, rl, 1, false, sm);
        grid_sync(a.flags, ++e);
      }
      // ---- attention: key-split partials, merged per row tile on its XCD ---------------
      attn_phase(a, pb, l, rl, sm, e + 1, gin_o(a, lw.o, rl));
      grid_sync(a.flags, ++e);
      // ---- O projection + gated residual -------------------------------------------------
      {
        const GemmIn g = gin_o(a, lw.o, rl);
        const GItem gi = gemm_item(g, 0);
        const bool has = gi.valid;
        V16 wr[2][kPCh];
        read_w(sm, wr, has ? 1 : 0, g.w8);
        V16 ra[kPCh][4];
        load_a(g, M, ra);
        const int tile = gi.tile;
        const int n = tile * 16 + 4 * eq;
        ResidIn rin;
        rin.issue(a, er, n, site(a, k, 2 * l, 2), site(a, k, 2 * l + 1, 0), has && gi.ks == 0 && t < 256, W8 ? lw.so : nullptr);
        f32x4 v[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if (has) gemm_core(wr, ra, sm, 1, v);
        else __syncthreads();   // as in gemm_core: every wave's read of wbuf is done
        prefetch_w(gin_up(a, lw.gu, rl), sm);
        if (has && split_reduce(a, g, e + 1, v[0]) && t < 256)
          epi_resid(a, v[0], rin, er, n, tile, rl + a.o_hsu, (float*)(rl + a.o_stu));
        grid_sync(a.flags, ++e);
      }
      // ---- gate / up + GELU(gate) * up ---------------------------------------------------
      {
        const GemmIn g = gin_up(a, lw.gu, rl);
        const int nslot = gemm_slots(g);
        V16 wr[2][kPCh];
        read_w(sm, wr, nslot, g.w8);
        V16 ra[kPCh][4];
        load_a(g, M, ra);
        StatLoad st;
        st.issue(rl + a.o_stu, M, D);
        V16 cv[2], wsv[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int n = ((int)blockIdx.x + s2 * G) * 16 + 4 * eq;   // interleaved (gate_f, up_f) pairs
          const bool use = t < 256 && s2 < nslot && er < M;
          cv[s2] = col4(cvec(a, k, 2 * l + 1), min(n, a.cg4 - 4), a.cg4, use);
          wsv[s2] = W8 ? col4(lw.sgu, min(n, a.cg4 - 4), a.cg4, use) : as_v(f32x4{1.f, 1.f, 1.f, 1.f});
        }
        st.finish(D, a.eps, sm);
        f32x4 v[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if (nslot) gemm_core(wr, ra, sm, nslot, v);
        __syncthreads();
        prefetch_w(gin_down(a, lw.down, rl), sm);
        const Rsrc ra2 = make_rsrc(rl + a.o_act, act_bytes(M, a.F));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int n = ((int)blockIdx.x + s2 * G) * 16 + 4 * eq;
          if (t < 256 && s2 < nslot && er < M) {
            const f32x4 y = sm.rinv[er] * (as_f4(wsv[s2]) * v[s2]) + as_f4(cv[s2]);
            st4(ra2, act_off(er, n / 2, a.F), pack_bf2(gelu_tanh(y[0]) * y[1], gelu_tanh(y[2]) * y[3]));
          }
        }
        grid_sync(a.flags, ++e);
      }
      // ---- down + gated residual (next norm: QKV of layer l + 1, or the final norm) -----
      {
        const GemmIn g = gin_down(a, lw.down, rl);
        const GItem gi = gemm_item(g, 0);
        const bool has = gi.valid;
        char* rnext = rot(a, kk, l + 1);
        V16 wr[2][kPCh];
        read_w(sm, wr, has ? 1 : 0, g.w8);
        V16 ra[kPCh][4];
        load_a(g, M, ra);
        const int tile = gi.tile;
        const int n = tile * 16 + 4 * eq;
        ResidIn rin;
        rin.issue(a, er, n, site(a, k, 2 * l + 1, 2), site(a, k, 2 * l + 2, 0), has && gi.ks == 0 && t < 256, W8 ? lw.sdown : nullptr);
        f32x4 v[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if (has) gemm_core(wr, ra, sm, 1, v);
        else __syncthreads();
        if (l + 1 < a.L) prefetch_w(gin_qkv(a, layer_w(a, l + 1).qkv, rnext), sm);
        else prefetch_w(gin_out(a, rnext), sm);
        if (has && split_reduce(a, g, e + 1, v[0]) && t < 256)
          epi_resid(a, v[0], rin, er, n, tile, rnext + a.o_hs, (float*)(rnext + a.o_st));
        grid_sync(a.flags, ++e);
      }
    }
    // ---- final norm + velocity projection + Euler update ---------------------------------
    {
      char* rf = rot(a, kk, a.L);
      const GemmIn g = gin_out(a, rf);
      const bool has = gemm_item(g, 0).valid;
      V16 wr[2][kPCh];
      read_w(sm, wr, has ? 1 : 0, g.w8);
      V16 ra[kPCh][4];
      load_a(g, M, ra);
      StatLoad st;
      st.issue(rf + a.o_st, M, D);
      const int n = (int)blockIdx.x * 16 + 4 * eq;
      const bool eok = has && t < 256 && er < M;
      const V16 cv = col4(cvec(a, k, 2 * a.L), min(n, a.cout4 - 4), a.cout4, eok);
      const V16 bo = col4(a.b_out, min(n, a.cout4 - 4), a.cout4, eok);
      V16 xo = ld16<kCpSc1>(rx, (eok && n < a.da) ? (uint32_t)((er * a.da + n) * 4) : kOob);
      const Rsrc rd = make_rsrc(a.dts, (uint32_t)(a.max_steps * 4));
      const float dt = __uint_as_float(ld4<0>(rd, (uint32_t)(k * 4)));
      st.finish(D, a.eps, sm);
      f32x4 v[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if (has) gemm_core(wr, ra, sm, 1, v);
      __syncthreads();
      if (kk + 1 < la.nsteps) prefetch_w(gin_qkv(a, layer_w(a, 0).qkv, rot(a, kk + 1, 0)), sm);
      if (eok) {
        const f32x4 vel = sm.rinv[er] * v[0] + as_f4(cv) + as_f4(bo);
        if (la.vout) {
          const Rsrc rv = make_rsrc(la.vout, (uint32_t)(M * a.da * 4));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n + j < a.da) st4(rv, (uint32_t)((er * a.da + n + j) * 4), __float_as_uint(vel[j]));
        } else {
          const f32x4 x4 = as_f4(xo);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n + j < a.da) st4(rx, (uint32_t)((er * a.da + n + j) * 4), __float_as_uint(x4[j] + dt * vel[j]));
        }
      }
      if (kk + 1 < la.nsteps) grid_sync(a.flags, ++e);
    }
  }
  wait_vm();   // no copy outlives the kernel
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
int loop_barriers(int L, int steps) { return steps * (5 * L + 2) - 1; }

const char* loop_check(const LoopShape& s, int num_cus) {
  if (s.dtype_bf16 != 1) return "bf16 only";
  if (s.dh != kDH) return "head_dim 256 only";
  if (s.M < 1 || s.M > 64) return "batch x horizon must be at most 64 rows";
  if (num_cus > kMaxGrid) return "more than 256 CUs";
  if (s.L < 1 || s.L > kMaxLayers) return "too many layers";
  if (s.D % 16 != 0 || s.D / 16 > num_cus) return "hidden must be a multiple of 16 and at most 16 x CUs";
  if (s.qd % 32 != 0 || s.D % 32 != 0 || s.F % 32 != 0) return "GEMM K dims must be multiples of 32";
  // the QKV, gate / up and output phases run unsplit over K = hidden (no split-K reduction):
  // one GEMM item covers at most kPKS of K
  if (s.D % 512 != 0 || s.D > kPKS) return "hidden must be a multiple of 512 and at most 1024";
  if (s.da % 4 != 0 || s.da > kMaxDa) return "action_dim must be a multiple of 4 and at most 32";
  const int G = num_cus;
  auto items = [&](int N, int K) { return ((N + 15) / 16) * ((K + kPKS - 1) / kPKS); };
  auto fits = [&](int N, int K) {
    const int nks = (K + kPKS - 1) / kPKS, ntiles = (N + 15) / 16;
    if (nks > 4) return false;
    // split-K: the splits of tile n in slots (n / 8) * nks + ks of XCD n % 8
    return nks == 1 ? ntiles <= 2 * G : ((ntiles + 7) / 8) * nks * 8 <= G && ntiles * nks <= kMaxSplitItems / 2;
  };
  if (!fits(s.qd + 2 * s.dh, s.D) || !fits(s.D, s.qd) || !fits(2 * s.F, s.D) || !fits(s.D, s.F) || !fits(s.da, s.D))
    return "a GEMM phase has more items than two per CU";
  if (items(s.D, s.qd) > kMaxSplitItems || items(s.D, s.F) > kMaxSplitItems) return "too many split items";
  const int RT = (s.nq * s.H + 63) / 64;
  const int TP = (s.P + 31) / 32, TS = (s.H + 31) / 32;
  const int SA = (TP + TS + 1) / 2;
  const int rtb = s.B * RT;
  // row tile rb on XCD rb % 8, its splits in slots (rb / 8) * SA + sp of that XCD
  if (SA > kMaxSA || rtb > kMaxRowTiles || rtb * SA > kMaxAttnItems || ((rtb + 7) / 8) * SA * 8 > G)
    return "attention items exceed the grid";
  return nullptr;
}

hipError_t loop_launch(const LoopArgs* a_dev, const LaunchArgs& la, int grid, bool w8, hipStream_t s) {
  const LoopArgs* p = a_dev;
  LaunchArgs l2 = la;
  void* args[] = {&p, &l2};
  if (w8) return hipLaunchCooperativeKernel((const void*)k_loop<true>, dim3(grid), dim3(kPT), args, 0, s);
  return hipLaunchCooperativeKernel((const void*)k_loop<false>, dim3(grid), dim3(kPT), args, 0, s);
}

}  // namespace fm
