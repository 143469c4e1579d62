// XCD-parallel denoise loop (pi0.5-shaped expert, bf16, at most 64 action rows): every Euler
// step of a chunk inside ONE cooperative launch of one workgroup per CU.
//
// The 256 CUs form 8 XCDs of 32; the CUs of one XCD share an L2 that is coherent among them,
// while the L2s of different XCDs are not coherent with each other. Each layer is therefore
// split across the XCDs as tensor parallelism splits it across devices, so that only two
// exchanges per layer cross XCDs:
//   - XCD x owns query head x: it computes that head's q and the (shared) k and v, the head's
//     attention over its request's keys, and that head's slice of the output projection,
//     a partial sum of the O projection over all hidden columns;
//   - XCD x owns MLP columns [F/8 x, F/8 (x + 1)): its gate/up projection and its slice of the
//     down projection, again a partial sum over all hidden columns.
// The partial sums of the 8 XCDs are added (reduce) column block by column block: XCD c adds
// block c of all eight, applies the gated residual to its share of the fp32 residual stream
// (kept in LDS by the CU that owns those rows and columns) and publishes its block of the next
// norm's bf16 operand h (1 + scale) with the block's row sums of squares (all-gather). Phases
// inside an XCD meet at XCD-local barriers (atomics in that XCD's L2); the cross-XCD waits are
// point to point (flags and counters at device scope), never a grid-wide barrier.
//
// Per layer: norm operand in -> QKV + RoPE -> attention key tiles -> merge of the tiles -> O
// partial -> reduce + residual -> norm operand in -> gate/up + GELU * up -> down partial ->
// reduce + residual. Weights stream through LDS ahead of use: waves 4-7 ("copy waves") issue
// buffer->LDS copies of the next phases' weights and key tiles whenever their LDS slot frees,
// and wait for them only where they are consumed; waves 0-3 ("store waves") do every global
// store, so their waits never include copies.
//
// Coherence rules: data exchanged between XCDs is written with sc1 (device-scope) stores; the
// partial sums, rewritten every layer, are read with sc1 loads; the norm operands live in
// per-(step, site) buffers written once per launch and read with ordinary loads (no stale L2
// line can exist: kernel start invalidates the L2s). XCD-local buffers are written with
// ordinary stores (the L1 writes through to the shared L2) and read with sc1 loads, which miss
// the reader's L1: those buffers are rewritten every layer, and a CU that did little else since
// its last read of one still holds that layer's lines in its L1 (an L1 invalidate does not serve:
// the workgroup-scope form drops nothing, and the agent-scope form also drops the L2's lines).
// Every global access goes through a buffer descriptor whose extent is the allocation, so an
// index past a buffer reads zeros or drops the store. Every wait is bounded (~2^20 polls): an
// expired wait records the fault word and lets the workgroup run on, so the launch ends.
#include "fm_common.h"
#include "fm_kernels.h"
#include "fm_xloop.h"

namespace fm {
namespace {

constexpr int kT = 512;                 // threads per workgroup: 8 waves
constexpr int kDH = 256;                // head dim
constexpr uint32_t kSpin = 1u << 20;
constexpr int kSc1 = 16;                // cache policy operand: sc1
constexpr uint32_t kOob = 0x80000000u;  // byte offset past every extent here
constexpr int kMaxDa = 32;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) XLoopArgs XA;
typedef const __attribute__((address_space(4))) XLayerW CXLayerW;

// ---------------------------------------------------------------------------------------
// Memory helpers
// ---------------------------------------------------------------------------------------
template <int POL> __device__ __forceinline__ V16 ld16(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL); }
template <int POL> __device__ __forceinline__ u32x2 ld8(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL); }
template <int POL> __device__ __forceinline__ uint32_t ld4(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL); }
template <int POL> __device__ __forceinline__ void st16(Rsrc r, uint32_t off, V16 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POL); }
template <int POL> __device__ __forceinline__ void st8(Rsrc r, uint32_t off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, POL); }
template <int POL> __device__ __forceinline__ void st4(Rsrc r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, POL); }
template <int POL> __device__ __forceinline__ void st2(Rsrc r, uint32_t off, uint16_t v) { __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, POL); }
__device__ __forceinline__ f32x4 as_f4(V16 v) { return __builtin_bit_cast(f32x4, v); }
__device__ __forceinline__ V16 as_v(f32x4 v) { return __builtin_bit_cast(V16, v); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) { return bf16_bits_rne(a) | (bf16_bits_rne(b) << 16); }

// device-scope flag accesses (polled: volatile, waited in place)
__device__ __forceinline__ uint32_t flag_ld(const uint32_t* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ void flag_st(uint32_t* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
// XCD-local counters: atomics executed in the XCD's L2 (no sc1).
// Non-returning L2 atomics (issue only: nothing waits for them)
__device__ __forceinline__ void l2_add_nr(uint32_t* p, uint32_t v) {
  asm volatile("global_atomic_add %0, %1, off" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void l2_max_nr(uint32_t* p, uint32_t v) {
  asm volatile("global_atomic_umax %0, %1, off" : : "v"(p), "v"(v) : "memory");
}
// Read of an XCD-local counter: a returning atomic, executed in the XCD's L2.
__device__ __forceinline__ uint32_t l2_read(uint32_t* p) {
  uint32_t v;
  asm volatile("global_atomic_or %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p), "v"(0u) : "memory");
  return v;
}
__device__ __forceinline__ void wait_all() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }
// 16 bytes per lane into LDS from data other CUs wrote during this launch: device scope (sc1),
// so that the read misses this CU's L1 (which may hold the same address from an earlier layer).
__device__ __forceinline__ void dma16_lds_fresh(const V16& desc, uint32_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen sc1 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(desc)
      : "memory");
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ bool copy_wave() { return wave_id() >= 4; }

// s_waitcnt vmcnt(n) for a run-time n < 64 (the count is an instruction immediate): this
// wave's vector memory operations, all but the n most recent, have completed (they complete
// in issue order).
__device__ __forceinline__ void vm_wait_le(int n) {
#define VMW(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 0xF) | (((k) >> 4) << 14) | (0x7 << 4) | (0xF << 8)); break;
  switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
    VMW(0) VMW(1) VMW(2) VMW(3) VMW(4) VMW(5) VMW(6) VMW(7) VMW(8) VMW(9) VMW(10) VMW(11) VMW(12) VMW(13)
    VMW(14) VMW(15) VMW(16) VMW(17) VMW(18) VMW(19) VMW(20) VMW(21) VMW(22) VMW(23) VMW(24) VMW(25) VMW(26)
    VMW(27) VMW(28) VMW(29) VMW(30) VMW(31) VMW(32) VMW(33) VMW(34) VMW(35) VMW(36) VMW(37) VMW(38) VMW(39)
    VMW(40) VMW(41) VMW(42) VMW(43) VMW(44) VMW(45) VMW(46) VMW(47) VMW(48) VMW(49) VMW(50) VMW(51) VMW(52)
    VMW(53) VMW(54) VMW(55) VMW(56) VMW(57) VMW(58) VMW(59) VMW(60) VMW(61) VMW(62) default: VMW(63)
  }
#undef VMW
}

// Byte offset of element (r, k) of a fragment-major activation operand with K columns: 16 x 32
// blocks of 1 KB (row block r / 16, k-chunk k / 32), row-block major; lane (r % 16) + 16 ((k %
// 32) / 8) of a block holds 8 consecutive k, so one MFMA operand fragment is one contiguous KB.
__device__ __forceinline__ uint32_t act_off(int r, int k, int K) {
  return (uint32_t)(((((r >> 4) * (K >> 5) + (k >> 5)) * 64 + (r & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7)) * 2);
}

// ---------------------------------------------------------------------------------------
// LDS: three slots for weights and key tiles, and this CU's share of the residual stream
// ---------------------------------------------------------------------------------------
struct XSmem {
  V16 slotA[4096];          // 64 KB: QKV, gate/up and output-projection weights; then their partial tiles
  V16 slotB[4096];          // 64 KB: attention key tiles; down weights (lower half); O / down partial tiles (upper half)
  V16 slotO[1024];          // 16 KB: O-projection weights
  float hkeep[2][128];      // residual h of rows 2 rank, 2 rank + 1, columns [D/8 x, D/8 (x + 1))
  float rinv[64];           // 1 / RMS of the norm operand's rows
  float2 pml[4][64];        // attention: (max, sum) of the second tile of the pair, per row
  int dead;                 // a wait of this workgroup expired: later waits return at once
};

// Constant-memory records, copied field by field
__device__ __forceinline__ XPair pair_at(XA& a, int p) { return XPair{a.pair[p].b, a.pair[p].j}; }
__device__ __forceinline__ XLayerW layer_at(XA& a, int l) {
  CXLayerW* p = (CXLayerW*)a.lw + l;
  return XLayerW{p->qkv, p->o, p->gu, p->down, p->sqkv, p->so, p->sgu, p->sdown};
}

// Who am I: XCD x (from the hardware), rank within the XCD (blockIdx / 8: the dispatcher deals a
// launch round-robin over the 8 XCDs, so the workgroups of one XCD are one residue class of
// blockIdx mod 8 and their blockIdx / 8 are 0..31).
struct Who { int x, r; };
// The attention's key-tile pair of a CU: pair p runs on rank 31 - p, so the pairs take the ranks
// with one QKV tile (16-31) and, at horizon <= 50 and batch 1, no rows of the reduce.
__device__ __forceinline__ int pair_of(const Who& me) { return 31 - me.r; }

// ---------------------------------------------------------------------------------------
// Waits
// ---------------------------------------------------------------------------------------
// Thread 0 polls an XCD-local word until it reaches target (bounded: an expired wait records
// `code` in the fault word and marks the workgroup dead, so later waits return at once). One
// lane only: the words are single L2 lines that every CU of the XCD polls.
__device__ __forceinline__ void local_wait(XA& a, uint32_t* p, uint32_t target, uint32_t code, XSmem& sm) {
  if (threadIdx.x == 0) {
    uint32_t n = 0;
    while (!sm.dead && l2_read(p) < target) {
      if (++n > kSpin) { flag_st(a.flags + kXErr, code); sm.dead = 1; }
    }
  }
}

// XCD barrier, in two halves so that copies can be issued between them without delaying the
// arrival. Arrive: every store wave's stores complete, then one arrival per workgroup on the
// XCD's counter, issued before anything the copy waves issue next (copy waves arrive without
// waiting for their copies: they store nothing). Wait: all 32 arrivals.
__device__ __forceinline__ void xarrive(XA& a, const Who& me) {
  if (!copy_wave()) wait_all();
  __syncthreads();
  if (threadIdx.x == 0) l2_add_nr(a.flags + kXBar + 32 * me.x, 1u);
  __syncthreads();
}
__device__ __forceinline__ void xwait(XA& a, const Who& me, uint32_t target, XSmem& sm) {
  local_wait(a, a.flags + kXBar + 32 * me.x, target, 1u, sm);
  __syncthreads();
}

// Cross-XCD waits are polled by one CU per XCD (rank kPoller), which then releases the others
// through an XCD-local word: the device-scope words see 8 pollers instead of 256, and the other
// CUs wait on their own L2.
constexpr int kPoller = 0;
__device__ __forceinline__ void xcd_release(XA& a, const Who& me, int rel, uint32_t target, uint32_t code, XSmem& sm) {
  uint32_t* p = a.flags + rel + 32 * me.x;
  if (me.r == kPoller) {
    if (threadIdx.x == 0) l2_max_nr(p, target);
  } else {
    local_wait(a, p, target, code, sm);
  }
  __syncthreads();
}

// Wait until every XCD's share of a norm operand is out (each XCD counter >= target).
__device__ __forceinline__ void ag_wait(XA& a, const Who& me, uint32_t target, XSmem& sm) {
  if (me.r == kPoller && threadIdx.x < 8 && !sm.dead) {
    const uint32_t* p = a.flags + kXAg + 32 * threadIdx.x;
    uint32_t n = 0;
    while (true) {
      const uint32_t v = flag_ld(p);
      if (__all(v >= target)) break;   // over the 8 active lanes
      if (++n > kSpin) { if (threadIdx.x == 0) { flag_st(a.flags + kXErr, 2u); sm.dead = 1; } break; }
    }
  }
  xcd_release(a, me, kXRelAg, target, 2u, sm);
}

// Wait until partial flags [rank][y] >= e for ranks r0..r0+3 and XCDs y < ny.
__device__ __forceinline__ void part_wait(XA& a, const Who& me, int base, int r0, int ny, uint32_t e, XSmem& sm) {
  if (me.r == kPoller && threadIdx.x < 32 && !sm.dead) {
    const int j = threadIdx.x >> 3, y = threadIdx.x & 7;
    const uint32_t* p = a.flags + base + (r0 + j) * 8 + y;
    uint32_t n = 0;
    while (true) {
      const uint32_t v = y < ny ? flag_ld(p) : 0xffffffffu;
      if (__all(v >= e)) break;   // over the 32 active lanes
      if (++n > kSpin) { if (threadIdx.x == 0) { flag_st(a.flags + kXErr, 3u); sm.dead = 1; } break; }
    }
  }
  xcd_release(a, me, base == kXFo ? kXRelO : kXRelD, e, 3u, sm);
}

// ---------------------------------------------------------------------------------------
// Weight prefetch: the copy waves copy this CU's fragments of a GEMM into an LDS slot. Tile s
// (of nt) is weight row block nb[s]; its chunks c0 .. c0 + nch of a matrix with kbw 32-wide
// k-chunks per row block. bf16: fragment (nb, kc) at ((nb kbw + kc) 64 + lane) 16 bytes, LDS
// (s nch + c) KB; FP8 (W8): one 1 KB fragment holds 16 rows x 64 k, at ((nb kbw/2 + kc/2) 64 +
// lane) 16, LDS (s nch/2 + c/2) KB. Returns the copies this wave issued.
// ---------------------------------------------------------------------------------------
template <bool W8>
__device__ __forceinline__ int prefetch_w(const void* W, uint32_t wbytes, int kbw, const int (&nb)[2], int nt, int c0,
                                          int nch, V16* slot) {
  const int lane = threadIdx.x & 63, cw = wave_id() - 4;
  if (cw < 0) return 0;
  V16 dw = make_desc(W, wbytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) dw[i] = __builtin_amdgcn_readfirstlane(dw[i]);
  const int per = W8 ? nch / 2 : nch;   // fragments per tile
  int issued = 0;
  for (int f = cw; f < nt * per; f += 4) {
    const int s = f / per, c = f % per;
    const uint32_t off = W8 ? (uint32_t)(((nb[s] * (kbw / 2) + c0 / 2 + c) * 64 + lane) * 16)
                            : (uint32_t)(((nb[s] * kbw + c0 + c) * 64 + lane) * 16);
    dma16_lds(dw, lds_addr(slot + (size_t)f * 64), off);
    ++issued;
  }
  return issued;
}

// ---------------------------------------------------------------------------------------
// GEMM of one phase: nt (1 or 2) tiles of 16 output columns over this CU's K range of nch
// 32-wide chunks, weights in LDS at `slot` (as prefetch_w put them), A fragment-major with kba
// chunks per row block starting at chunk c0, M <= 64 rows. nw waves take part (8, or 4: waves
// 0-3 only; the others return zeros at once): wave w takes chunk pairs w and w + nw. Partial
// tiles are summed through `red` (which may be `slot` itself: every wave has read its weights
// before any partial is written). Thread t < 256 ends with v[s] = row t / 4,
// columns 4 (t % 4) .. + 3 of tile s. Every participating wave has passed two __syncthreads.
// ---------------------------------------------------------------------------------------
template <bool W8, int APOL = 0>
__device__ __forceinline__ void xgemm(const char* A, uint32_t abytes, int kba, int c0, int nch, int M, int nt, int nw,
                                      const V16* slot, float* red, f32x4 (&v)[2]) {
  typedef Mma<bf16>::frag frag;
  const int lane = threadIdx.x & 63, w = wave_id();
  const bool part = w < nw && nt > 0;
  // chunks of this wave: 2 (w + nw p) + {0, 1}, p < 2 (an FP8 fragment holds a chunk pair).
  // bf16 weights take the same assignment, so that a GEMM over FP8 codes and one over the
  // dequantized bf16 weights add the same partial tiles in the same order: with a power-of-two
  // row scale applied after the sum, the two are then bitwise equal.
  int cj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cj[j] = 2 * (w + nw * (j >> 1)) + (j & 1);
  V16 wr[2][4], ra[4][4];
  const Rsrc rA = make_rsrc(A, abytes);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int row = 16 * mb + (lane & 15);
      ra[j][mb] = ld16<APOL>(rA, (part && cj[j] < nch && row < M) ? (uint32_t)(((mb * kba + c0 + cj[j]) * 64 + lane) * 16) : kOob);
    }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (W8) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c = cj[2 * p];
        const V16 x = (part && s < nt && c < nch) ? slot[(s * (nch / 2) + c / 2) * 64 + lane] : vzero();
        wr[s][2 * p] = fp8x8_bf16(x[0], x[1]);
        wr[s][2 * p + 1] = fp8x8_bf16(x[2], x[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) wr[s][j] = (part && s < nt && cj[j] < nch) ? slot[(s * nch + cj[j]) * 64 + lane] : vzero();
    }
  }
  __syncthreads();   // every wave holds its weights: `red` may overwrite the slot
  f32x4 acc[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[s][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (part) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        acc[0][mb] = Mma<bf16>::mma(__builtin_bit_cast(frag, ra[j][mb]), __builtin_bit_cast(frag, wr[0][j]), acc[0][mb]);
        if (nt > 1) acc[1][mb] = Mma<bf16>::mma(__builtin_bit_cast(frag, ra[j][mb]), __builtin_bit_cast(frag, wr[1][j]), acc[1][mb]);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s >= nt) break;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((s * nw + w) * 64 + 16 * mb + 4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[s][mb][e];
    }
  }
  __syncthreads();
  const int t = threadIdx.x, r = (t & 255) >> 2, q = t & 3;
  v[0] = v[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (t < 256) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s >= nt) break;
      for (int ww = 0; ww < nw; ++ww) v[s] += *(const f32x4*)&red[((s * nw + ww) * 64 + r) * 16 + 4 * q];
    }
  }
  __syncthreads();   // every read of `red` is done: the slot may take new copies
}

// 16 bytes of a per-column fp32 vector at column n (padded to 4 floats); zeros without a
// memory access where ok is false
__device__ __forceinline__ V16 col4(const float* p, int n, int limit, bool ok = true) {
  const Rsrc r = make_rsrc(p, (uint32_t)(limit * 4));
  return ld16<0>(r, ok ? (uint32_t)(n * 4) : kOob);
}

// 1 / RMS of the norm operand's rows into LDS: row m's eight block sums of squares.
__device__ __forceinline__ void load_rinv(XA& a, const char* agst, XSmem& sm) {
  const int t = threadIdx.x;
  if (t < 64) {
    const Rsrc rs = make_rsrc(agst, 64 * 8 * 4);
    const bool ok = t < a.M;
    const f32x4 p0 = as_f4(ld16<0>(rs, ok ? (uint32_t)(t * 32) : kOob));
    const f32x4 p1 = as_f4(ld16<0>(rs, ok ? (uint32_t)(t * 32 + 16) : kOob));
    const float ss = ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
    sm.rinv[t] = rsqrtf(ss / (float)a.D + a.eps);
  }
}

// ---------------------------------------------------------------------------------------
// Reduce (and the in-projection): CU (x, rank) owns rows 2 rank, 2 rank + 1 and columns
// [D/8 x, D/8 (x + 1)) of the residual stream. It adds the XCDs' partial sums of those columns,
// applies the gated residual, and publishes its block of the next norm's bf16 operand
// h (1 + scale) and the rows' sums of squares over the block, then one arrival on the XCD's
// norm-operand counter. Threads: 4 columns each, D/32 per row.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void publish(XA& a, const Who& me, char* agbuf, int tpr, int rs, int m, int n, bool ok,
                                        f32x4 h, const f32x4& sc) {
  float ss = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
  // sum over the row's tpr (16 or 32) consecutive lanes
  ss = group_sum<16>(ss);
  if (tpr == 32) ss += __shfl_xor(ss, 16);
  if (ok) {
    const Rsrc rh = make_rsrc(agbuf, (uint32_t)a.o_agst);
    st8<kSc1>(rh, act_off(m, n, a.D),
              u32x2{pack_bf2(h[0] * (1.f + sc[0]), h[1] * (1.f + sc[1])), pack_bf2(h[2] * (1.f + sc[2]), h[3] * (1.f + sc[3]))});
    if ((threadIdx.x & (tpr - 1)) == 0) {
      const Rsrc rt = make_rsrc(agbuf + a.o_agst, 64 * 8 * 4);
      st4<kSc1>(rt, (uint32_t)((m * 8 + me.x) * 4), __float_as_uint(ss));
    }
  }
  (void)rs;
}
__device__ __forceinline__ void ag_arrive(XA& a, const Who& me) {
  if (!copy_wave()) wait_all();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(a.flags + kXAg + 32 * me.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------
// Attention of one key-tile pair: CU rank 31 - p of XCD x takes pair p of head x; the waves of half h
// (waves 4 h .. 4 h + 3) take tile j + h of the pair, wave w4 the query rows 16 w4 .. + 15 of the
// request. S^T = K Q^T and O^T = V^T P^T on MFMA with the tile's K / V^T in LDS (32 KB at
// slotB + 32 KB h). The two halves are merged in LDS, and the pair's unnormalised output O
// (rows < H, row-major [row][256] fp32) and each row's (max, sum) are stored for the merge.
// ---------------------------------------------------------------------------------------
constexpr int kDCH = kDH / 32, kDB = kDH / 16;
constexpr int kFK = 2 * kDCH, kFT = kFK + kDB;   // K and V^T fragments of one key tile

// number of key tiles of request b
__device__ __forceinline__ int req_tiles(XA& a, int b) { return (a.plen[b] + 31) / 32 + (a.H + 31) / 32; }

// Copies of half h's key tile into LDS (this wave does fragments f = w + 4 i of the 32): prefix
// tiles from the pool when suffix == false, the chunk's own tiles from this step's K / V^T when
// suffix == true. Returns the copies issued.
__device__ __forceinline__ int tile_issue(XA& a, const Who& me, int l, int h, bool suffix, int w, XSmem& sm) {
  const int p = pair_of(me);
  if (p >= a.npairs) return 0;
  const int lane = threadIdx.x & 63;
  const XPair pr = pair_at(a, p);
  const int b = pr.b, j = pr.j + h, tp = (a.plen[b] + 31) / 32;
  if (j >= req_tiles(a, b)) return 0;
  const bool is_suf = j >= tp;
  if (is_suf != suffix) return 0;
  V16 dk, dv;
  int kt, vds;
  if (!is_suf) {
    const bf16* kp = a.pool + (size_t)(2 * l) * a.plane + (size_t)b * a.cap * kDH;
    const bf16* vp = a.pool + (size_t)(2 * l + 1) * a.plane + (size_t)b * kDH * a.cap;
    dk = make_desc(kp, (uint32_t)(a.cap * kDH * 2));
    dv = make_desc(vp, (uint32_t)(kDH * a.cap * 2));
    kt = 32 * j; vds = a.cap;
  } else {
    const char* xl = a.xl + (size_t)me.x * a.xl_stride;
    dk = make_desc(xl + a.o_sk + (size_t)b * a.Hp * kDH * 2, (uint32_t)(a.Hp * kDH * 2));
    dv = make_desc(xl + a.o_svt + (size_t)b * kDH * a.Hp * 2, (uint32_t)(kDH * a.Hp * 2));
    kt = 32 * (j - tp); vds = a.Hp;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) { dk[u] = __builtin_amdgcn_readfirstlane(dk[u]); dv[u] = __builtin_amdgcn_readfirstlane(dv[u]); }
  const uint32_t lds0 = lds_addr(&sm.slotB[h * 2048]);
  int issued = 0;
  for (int f = w; f < kFT; f += 4) {
    uint32_t off;
    if (is_suf) {   // fragment-major: contiguous kilobytes
      if (f < kFK) off = (uint32_t)(((((kt >> 4) + f / kDCH) * kDCH + f % kDCH) * 64 + lane) * 16);
      else off = (uint32_t)((((f - kFK) * (vds >> 5) + (kt >> 5)) * 64 + lane) * 16);
    } else if (f < kFK) {
      off = (uint32_t)(((kt + 16 * (f / kDCH) + (lane & 15)) * kDH + (f % kDCH) * 32 + (lane >> 4) * 8) * 2);
    } else {
      off = (uint32_t)(((16 * (f - kFK) + (lane & 15)) * vds + kt + (lane >> 4) * 8) * 2);
    }
    if (is_suf) dma16_lds_fresh(f < kFK ? dk : dv, lds0 + (uint32_t)f * 1024u, off);
    else dma16_lds(f < kFK ? dk : dv, lds0 + (uint32_t)f * 1024u, off);
    ++issued;
  }
  return issued;
}

__device__ __forceinline__ void attn_pair(XA& a, const Who& me, XSmem& sm) {
  typedef Mma<bf16>::frag frag;
  const int lane = threadIdx.x & 63, w = wave_id(), w4 = w & 3, h = w >> 2;
  const int pi = pair_of(me);
  const bool valid = pi < a.npairs;
  const XPair pr = valid ? pair_at(a, pi) : XPair{0, 0};
  const int b = pr.b, j = pr.j + h, tp = (a.plen[b] + 31) / 32;
  const bool has = valid && j < req_tiles(a, b) && 16 * w4 < a.H;   // a tile and query rows for this wave
  const bool is_suf = j >= tp;
  const int kbase = is_suf ? 32 * (j - tp) : 32 * j;
  const int klim = is_suf ? a.H : a.plen[b];
  const char* xl = a.xl + (size_t)me.x * a.xl_stride;
  f32x4 o[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // a half without a tile keeps (O, l) = 0 and a finite reference below any score, which the
  // merge below weighs by exp2(-1e30 - m) = 0
  float m = -1e30f, lsum = 0.f;
  if (has) {
    frag qf[kDCH];
    const Rsrc rq = make_rsrc(xl + a.o_q, (uint32_t)(a.B * 64 * kDH * 2));
    const int blk = b * 4 + w4;
#pragma unroll
    for (int c = 0; c < kDCH; ++c) qf[c] = __builtin_bit_cast(frag, ld16<kSc1>(rq, (uint32_t)(((blk * kDCH + c) * 64 + lane) * 16)));
    const V16* sK = &sm.slotB[h * 2048];
    const V16* sV = sK + kFK * 64;
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
      for (int c = 0; c < kDCH; c += 2) {
        s0 = Mma<bf16>::mma(__builtin_bit_cast(frag, sK[(kb * kDCH + c) * 64 + lane]), qf[c], s0);
        s1 = Mma<bf16>::mma(__builtin_bit_cast(frag, sK[(kb * kDCH + c + 1) * 64 + lane]), qf[c + 1], s1);
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
    m = group4_max(mt);   // the tile has a visible key: m is finite
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
    for (int db = 0; db < kDB; ++db) o[db] = Mma<bf16>::mma(__builtin_bit_cast(frag, sV[db * 64 + lane]), pf, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  __syncthreads();   // every wave has read its key tile: slotB takes the second half's result
  f32x4* mrg = (f32x4*)sm.slotB;   // [w4][db][lane]
  if (h == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db) mrg[(w4 * kDB + db) * 64 + lane] = o[db];
    sm.pml[w4][lane] = make_float2(m, lsum);
  }
  __syncthreads();
  if (h == 0 && valid && 16 * w4 < a.H) {
    const float2 p2 = sm.pml[w4][lane];
    const float mx = fmaxf(m, p2.x);
    const float a1 = exp2f(m - mx), a2 = exp2f(p2.x - mx);
    const int row = 16 * w4 + (lane & 15);
    if (row < a.H) {
      const Rsrc rw = make_rsrc(xl + a.o_ap, (uint32_t)(a.npairs * 64 * kDH * 4));
      const uint32_t rb = (uint32_t)((pi * 64 + row) * kDH * 4);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const f32x4 v = a1 * o[db] + a2 * mrg[(w4 * kDB + db) * 64 + lane];
        st16<0>(rw, rb + (uint32_t)((16 * db + 4 * (lane >> 4)) * 4), as_v(v));
      }
      if (lane < 16) {
        const Rsrc rm = make_rsrc(xl + a.o_ml, (uint32_t)(a.npairs * 64 * 8));
        st8<0>(rm, (uint32_t)((pi * 64 + row) * 8), u32x2{__float_as_uint(mx), __float_as_uint(a1 * lsum + a2 * p2.y)});
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ XA& launder(const XLoopArgs* p) {
  XA* q = (XA*)p;
  asm volatile("" : "+s"(q));
  return *q;
}

template <bool W8>
__global__ void __launch_bounds__(kT, 1) k_xloop(const XLoopArgs* __restrict__ pa, XLaunch la) {
  __shared__ XSmem sm;
  const int t = threadIdx.x, w = wave_id();
  const int er = (t & 255) >> 2, eq = t & 3;   // epilogue thread: row, 4-column run
  // a fault word left by an earlier launch: its results were invalid and so are this launch's
  // inputs; write NaN where the result goes and stop, every workgroup alike
  if (flag_ld(pa->flags + kXErr) != 0u) {
    if (blockIdx.x == 0) {
      XA& a = launder(pa);
      float* dst = la.vout ? la.vout : la.xout;
      const Rsrc rd = make_rsrc(dst, (uint32_t)(a.M * a.da * 4));
      for (int i = t; i < a.M * a.da; i += kT) st4<kSc1>(rd, (uint32_t)(i * 4), 0x7fc00000u);
    }
    return;
  }
  const Who me = {(int)hw_xcc_id() & 7, (int)(blockIdx.x >> 3)};
  uint32_t nxb = 0, nag = 0, npe = 0;   // XCD barriers, norm operands, partial exchanges so far
  auto xa = [&](XA& a) { ++nxb; xarrive(a, me); };
  auto xw = [&](XA& a) { xwait(a, me, la.xb0 + 32u * nxb, sm); };
  auto xb = [&](XA& a) { xa(a); xw(a); };
  const bool has_head = me.x < pa->nq;
  const bool acu = has_head && pair_of(me) < pa->npairs;   // this CU takes a key-tile pair of the attention

  // copy-wave bookkeeping: this wave's gate/up, down, next-QKV and prefix-tile copies not yet
  // waited for
  int c_gu = 0, c_dn = 0, c_qk = 0, c_tl = 0;
  // copy waves of a CU with a tile pair: layer l's prefix key tiles into slot B. The prefix is
  // bound for the whole chunk, so they are issued a phase group early: after the previous
  // layer's down GEMM (or with the first layer's QKV weights), and land during the reduce and
  // the QKV phase; the attention waits for them.
  auto issue_tiles = [&](XA& a, int l) {
    c_tl = 0;
    if (copy_wave() && acu) c_tl = tile_issue(a, me, l, 0, false, wave_id() - 4, sm) + tile_issue(a, me, l, 1, false, wave_id() - 4, sm);
  };

  // (XCD, rank) slot check: two workgroups on one slot mean the dispatch was not round-robin
  if (t == 0) sm.dead = 0;
  {
    XA& a = launder(pa);
    if (t == 0) a.flags[kXSlot + 32 * me.x + me.r] = blockIdx.x;   // ordinary store: XCD-local
    xb(a);
    if (t == 0 && *(volatile const uint32_t*)&a.flags[kXSlot + 32 * me.x + me.r] != blockIdx.x) {
      flag_st(a.flags + kXErr, kXFaultSlot);
      sm.dead = 1;
    }
    __syncthreads();
  }

  for (int kk = 0; kk < la.nsteps; ++kk) {
    XA& a = launder(pa);
    const int k = la.k0 + kk;
    const int D = a.D, M = a.M, bw = D / 8;          // block width of the reduce
    const int tpr = bw / 4;                           // reduce threads per row
    char* xl = a.xl + (size_t)me.x * a.xl_stride;
    auto agb = [&](int site) { return a.ag + (size_t)kk * a.ag_step + (size_t)site * a.ag_site; };
    auto site_v = [&](int s, int part) { return a.table + ((size_t)k * a.S + s) * 3 * D + (size_t)part * D; };
    auto cvec = [&](int s) {
      const long off = s == 2 * a.L ? (long)a.L * (a.cq4 + a.cg4) : (long)(s / 2) * (a.cq4 + a.cg4) + (s % 2) * a.cq4;
      return a.cbuf + (size_t)k * a.csum + off;
    };
    // weight row blocks of this CU's tiles
    auto qkv_nb = [&](int tt) { return tt < 16 ? 16 * me.x + tt : (tt < 32 ? 16 * a.nq + tt - 16 : 16 * a.nq + 16 + tt - 32); };
    const int nt_q = me.r + 32 < 48 ? 2 : 1;   // QKV tiles: r and r + 32 of the head's 48
    const int nqkv[2] = {qkv_nb(me.r), qkv_nb(me.r + 32 < 48 ? me.r + 32 : me.r)};
    const int gut = a.F / 64;                   // gate/up tiles of this XCD
    const int nt_g = me.r < gut ? (me.r + 32 < gut ? 2 : 1) : 0;
    const int ngu[2] = {(a.F / 64) * me.x + me.r, (a.F / 64) * me.x + me.r + 32};
    const int nt_od = D / 512;                  // O and down tiles of this CU (16 D/512 columns)
    const int nod[2] = {me.r * nt_od, me.r * nt_od + 1};
    const int nt_out = me.r * 16 < a.da ? 1 : 0;
    const int nout[2] = {me.r, me.r};

    // ---- in-projection: h = x W_in^T + b_in for this CU's rows and block; the chunk x of the
    // first step is copied into this XCD's x buffer (later steps' x is written there) --------
    {
      const int rs = t / tpr, m = 2 * me.r + rs, n = bw * me.x + 4 * (t % tpr);
      const bool ok = t < 2 * tpr && m < M;
      const Rsrc rxi = make_rsrc(kk == 0 ? la.xin : (const float*)(xl + a.o_xx), (uint32_t)(M * a.da * 4));
      const Rsrc rw = make_rsrc(a.w_in, (uint32_t)(D * a.da * 2));
      V16 xv[kMaxDa / 4];
      u32x2 wv[4][kMaxDa / 4];
#pragma unroll
      for (int j = 0; j < kMaxDa / 4; ++j) {
        const bool in = 4 * j < a.da;
        const uint32_t off = (ok && in) ? (uint32_t)((m * a.da + 4 * j) * 4) : kOob;
        xv[j] = ld16<kSc1>(rxi, off);
#pragma unroll
        for (int c = 0; c < 4; ++c) wv[c][j] = ld8<0>(rw, (ok && in) ? (uint32_t)(((n + c) * a.da + 4 * j) * 2) : kOob);
      }
      const V16 bb = col4(a.b_in, n, D, ok);
      const V16 sc = col4(site_v(0, 0), n, D, ok);
      f32x4 h = as_f4(bb);
#pragma unroll
      for (int j = 0; j < kMaxDa / 4; ++j) {
        const f32x4 x4 = as_f4(xv[j]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float wf[4] = {__uint_as_float(wv[c][j][0] << 16), __uint_as_float(wv[c][j][0] & 0xffff0000u),
                               __uint_as_float(wv[c][j][1] << 16), __uint_as_float(wv[c][j][1] & 0xffff0000u)};
#pragma unroll
          for (int u = 0; u < 4; ++u) h[c] += x4[u] * wf[u];
        }
      }
      if (t < 2 * tpr) {
        if (kk == 0 && ok && (t % tpr) == 0) {   // this XCD's copy of x: the row's first thread
          const Rsrc rxx = make_rsrc(xl + a.o_xx, (uint32_t)(M * a.da * 4));
#pragma unroll
          for (int j = 0; j < kMaxDa / 4; ++j)
            if (4 * j < a.da) st16<0>(rxx, (uint32_t)((m * a.da + 4 * j) * 4), xv[j]);
        }
        *(f32x4*)&sm.hkeep[rs][4 * (t % tpr)] = h;
        publish(a, me, agb(0), tpr, rs, m, n, ok, h, as_f4(sc));
      }
      ag_arrive(a, me);
      ++nag;
      // copy waves: the first layer's QKV weights and prefix key tiles, behind the arrival
      __syncthreads();
      if (copy_wave() && has_head)
        prefetch_w<W8>(layer_at(a, 0).qkv, a.wb_qkv, D / 32, nqkv, nt_q, 0, D / 32, sm.slotA);
      issue_tiles(a, 0);
    }

    for (int l = 0; l < a.L; ++l) {
      XA& a = launder(pa);
      const XLayerW lw = layer_at(a, l);
      const int sq = 2 * l, su = 2 * l + 1, sn = 2 * l + 2;   // norm sites: QKV, gate/up, next
      // ================= QKV + RoPE (XCD x: head x's q, and k, v) =================
      if (copy_wave()) vm_wait_le(c_tl);   // this layer's QKV weights have landed (the key tiles may fly)
      ag_wait(a, me, la.ag0 + 32u * nag, sm);
      {
        char* ab = agb(sq);
        load_rinv(a, ab + a.o_agst, sm);
        // epilogue inputs of both tiles, in flight during the GEMM: c of the folded norm, the
        // FP8 row scales, RoPE cos / sin
        const bool eok = has_head && t < 256 && er < M;
        V16 ecv[2], ews[2], ecs[2];
        int eG[2], ed[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int tt = s2 == 0 ? me.r : me.r + 32;
          const bool use = eok && s2 < nt_q;
          ed[s2] = (tt & 15) * 16 + 4 * eq;
          eG[s2] = tt < 16 ? me.x * kDH + ed[s2] : (tt < 32 ? a.nq * kDH + ed[s2] : a.nq * kDH + kDH + ed[s2]);
          ecv[s2] = col4(cvec(sq), eG[s2], a.cq4, use);
          ews[s2] = W8 ? col4(lw.sqkv, eG[s2], a.cq4, use) : as_v(f32x4{1.f, 1.f, 1.f, 1.f});
          const Rsrc rc = make_rsrc(a.rope_cs, (uint32_t)(a.B * a.H * (kDH / 2) * 8));
          ecs[s2] = ld16<0>(rc, (use && a.rope && tt < 32) ? (uint32_t)((er * (kDH / 2) + ed[s2] / 2) * 8) : kOob);
        }
        f32x4 v[2];
        xgemm<W8>(ab, (uint32_t)a.o_agst, D / 32, 0, D / 32, M, has_head ? nt_q : 0, 8, sm.slotA, (float*)sm.slotA, v);
        if (eok) {
          const int b = er / a.H, i = er % a.H;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 >= nt_q) break;
            const int tt = s2 == 0 ? me.r : me.r + 32;
            const int d = ed[s2];                             // column within q, k or v
            f32x4 y = sm.rinv[er] * (as_f4(ews[s2]) * v[s2]) + as_f4(ecv[s2]);
            if (a.rope && tt < 32) {
              const f32x4 cs = as_f4(ecs[s2]);
              const float x0 = y[0], x1 = y[1], x2 = y[2], x3 = y[3];
              y[0] = x0 * cs[0] - x1 * cs[1];
              y[1] = x1 * cs[0] + x0 * cs[1];
              y[2] = x2 * cs[2] - x3 * cs[3];
              y[3] = x3 * cs[2] + x2 * cs[3];
            }
            const u32x2 pk = u32x2{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
            if (tt < 16) {
              const Rsrc rq = make_rsrc(xl + a.o_q, (uint32_t)(a.B * 64 * kDH * 2));
              st8<0>(rq, act_off(b * 64 + i, d, kDH), pk);
            } else if (tt < 32) {
              const Rsrc rk = make_rsrc(xl + a.o_sk, (uint32_t)(a.B * a.Hp * kDH * 2));
              st8<0>(rk, act_off(b * a.Hp + i, d, kDH), pk);
            } else {
              const Rsrc rv = make_rsrc(xl + a.o_svt, (uint32_t)(a.B * kDH * a.Hp * 2));
              const int slot = vt_slot<bf16>(i);
#pragma unroll
              for (int j = 0; j < 4; ++j) st2<0>(rv, act_off(b * kDH + d + j, slot, a.Hp), __builtin_bit_cast(uint16_t, (bf16)y[j]));
            }
          }
        }
        // A CU's vector memory operations complete in issue order, whichever wave issued them,
        // and the weight streams of all CUs share the XCD's L2 and the HBM: copies are issued
        // after each phase's own loads, stores and barrier arrival, one phase's worth at a time.
        // Copy waves: this layer's O weights.
        xa(a);
        if (copy_wave() && has_head)
          prefetch_w<W8>(lw.o, a.wb_o, a.nq * kDH / 32, nod, nt_od, me.x * (kDH / 32), kDH / 32, sm.slotO);
        xw(a);
      }
      // ================= attention: pair me.r of head x (a CU with a pair) =================
      {
        // the chunk's own key tiles are this phase's inputs; the prefix tiles were copied
        // since the previous layer's down GEMM
        if (acu) {
          tile_issue(a, me, l, w >> 2, true, w & 3, sm);
          wait_all();
          __syncthreads();
          attn_pair(a, me, sm);
        }
        xb(a);
      }
      // ================= merge of a head's key-tile pairs: rows 2 rank, 2 rank + 1 ==========
      {
        // wave rs < 2 merges row 2 rank + rs; lane g: dims 4 g .. 4 g + 3; each pair's row is
        // one contiguous kilobyte
        if (has_head && t < 128) {
          const int rs = t >> 6, m = 2 * me.r + rs, g = t & 63;
          if (m < M) {   // wave-uniform
            const int b = m / a.H, i = m % a.H, p0 = a.poff[b], np = a.poff[b + 1] - p0;
            const Rsrc rm = make_rsrc(xl + a.o_ml, (uint32_t)(a.npairs * 64 * 8));
            const u32x2 ml = ld8<kSc1>(rm, g < np ? (uint32_t)(((p0 + g) * 64 + i) * 8) : kOob);
            const float mu = g < np ? __uint_as_float(ml[0]) : -INFINITY;
            float mx = mu;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const float wu = g < np ? exp2f(mu - mx) : 0.f;
            float den = wu * __uint_as_float(ml[1]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
            const float wn = wu / den;
            const Rsrc rw = make_rsrc(xl + a.o_ap, (uint32_t)(a.npairs * 64 * kDH * 4));
            f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int u0 = 0; u0 < np; u0 += 16) {
              V16 ov[16];
#pragma unroll
              for (int u = 0; u < 16; ++u)
                ov[u] = ld16<kSc1>(rw, u0 + u < np ? (uint32_t)((((p0 + u0 + u) * 64 + i) * kDH + 4 * g) * 4) : kOob);
#pragma unroll
              for (int u = 0; u < 16; ++u) num += __shfl(wn, u0 + u) * as_f4(ov[u]);
            }
            const Rsrc rax = make_rsrc(xl + a.o_ax, (uint32_t)(64 * kDH * 2));
            st8<0>(rax, act_off(m, 4 * g, kDH), u32x2{pack_bf2(num[0], num[1]), pack_bf2(num[2], num[3])});
          }
        }
        // copy waves: this layer's gate/up weights (slot A is free since the QKV GEMM)
        xa(a);
        c_gu = copy_wave() && nt_g > 0 ? prefetch_w<W8>(lw.gu, a.wb_gu, D / 32, ngu, nt_g, 0, D / 32, sm.slotA) : 0;
        xw(a);
      }
      // ================= O projection: head x's slice, partial sums over all hidden columns ==
      {
        if (copy_wave()) vm_wait_le(c_gu);   // O weights landed (and the key tiles)
        __syncthreads();
        V16 ews[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          ews[s2] = W8 ? col4(lw.so, nod[s2] * 16 + 4 * eq, D, has_head && t < 256 && er < M && s2 < nt_od)
                       : as_v(f32x4{1.f, 1.f, 1.f, 1.f});
        f32x4 v[2];
        xgemm<W8, kSc1>(xl + a.o_ax, (uint32_t)(64 * kDH * 2), kDH / 32, 0, kDH / 32, M, has_head ? nt_od : 0, 4, sm.slotO,
                  (float*)&sm.slotB[2048], v);
        if (has_head && t < 256 && er < M) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 >= nt_od) break;
            const int n = nod[s2] * 16 + 4 * eq;
            const V16 wsv = ews[s2];
            const Rsrc rp = make_rsrc(a.part + (size_t)me.x * 64 * D, (uint32_t)(64 * D * 4));
            st16<kSc1>(rp, (uint32_t)((er * D + n) * 4), as_v(as_f4(wsv) * v[s2]));
          }
        }
        if (!copy_wave()) wait_all();
        __syncthreads();
        ++npe;
        if (t == 0 && has_head) flag_st(a.flags + kXFo + me.r * 8 + me.x, la.pe0 + npe);
        // copy waves: this layer's down weights (slot B's lower half), behind the flag
        __syncthreads();
        c_dn = copy_wave() ? prefetch_w<W8>(lw.down, a.wb_down, a.F / 32, nod, nt_od, me.x * (a.F / 256), a.F / 256, sm.slotB) : 0;
      }
      // ================= reduce the O partials + gated residual; publish the MLP's norm operand
      {
        part_wait(a, me, kXFo, 4 * me.x, a.nq < 8 ? a.nq : 8, la.pe0 + npe, sm);
        if (t < 2 * tpr) {
          const int rs = t / tpr, m = 2 * me.r + rs, n = bw * me.x + 4 * (t % tpr);
          const bool ok = m < M;
          const V16 g = col4(site_v(sq, 2), n, D, ok);
          const V16 sc = col4(site_v(su, 0), n, D, ok);
          const int ny = a.nq < 8 ? a.nq : 8;
          V16 p[8];
#pragma unroll
          for (int y = 0; y < 8; ++y) {
            const Rsrc rp = make_rsrc(a.part + (size_t)y * 64 * D, (uint32_t)(64 * D * 4));
            p[y] = ld16<kSc1>(rp, (ok && y < ny) ? (uint32_t)((m * D + n) * 4) : kOob);
          }
          f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int y = 0; y < 8; ++y) sum += as_f4(p[y]);
          f32x4 h = *(f32x4*)&sm.hkeep[rs][4 * (t % tpr)];
          h += as_f4(g) * sum;
          *(f32x4*)&sm.hkeep[rs][4 * (t % tpr)] = h;
          publish(a, me, agb(su), tpr, rs, m, n, ok, h, as_f4(sc));
        }
        ag_arrive(a, me);
        ++nag;
      }
      // ================= gate / up + GELU(gate) * up: XCD x's MLP columns ====================
      {
        if (copy_wave()) vm_wait_le(c_dn);   // gate/up weights landed (down weights may still fly)
        ag_wait(a, me, la.ag0 + 32u * nag, sm);
        char* ab = agb(su);
        load_rinv(a, ab + a.o_agst, sm);
        const bool eok = t < 256 && er < M;
        V16 ecv[2], ews[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int n = ngu[s2] * 16 + 4 * eq;   // interleaved (gate_f, up_f) column pairs
          const bool use = eok && s2 < nt_g;
          ecv[s2] = col4(cvec(su), n, a.cg4, use);
          ews[s2] = W8 ? col4(lw.sgu, n, a.cg4, use) : as_v(f32x4{1.f, 1.f, 1.f, 1.f});
        }
        f32x4 v[2];
        xgemm<W8>(ab, (uint32_t)a.o_agst, D / 32, 0, D / 32, M, nt_g, 8, sm.slotA, (float*)sm.slotA, v);
        if (eok) {
          const Rsrc ract = make_rsrc(xl + a.o_act, (uint32_t)(64 * (a.F / 8) * 2));
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 >= nt_g) break;
            const int n = ngu[s2] * 16 + 4 * eq;
            const f32x4 y = sm.rinv[er] * (as_f4(ews[s2]) * v[s2]) + as_f4(ecv[s2]);
            const int f = n / 2 - (a.F / 8) * me.x;   // column of this XCD's activation block
            st4<0>(ract, act_off(er, f, a.F / 8), pack_bf2(gelu_tanh(y[0]) * y[1], gelu_tanh(y[2]) * y[3]));
          }
        }
        // copy waves: the next layer's QKV weights, or the output projection's after the last
        // layer (slot A is free again)
        xa(a);
        c_qk = 0;
        if (copy_wave()) {
          if (l + 1 < a.L) {
            if (has_head) c_qk = prefetch_w<W8>(layer_at(a, l + 1).qkv, a.wb_qkv, D / 32, nqkv, nt_q, 0, D / 32, sm.slotA);
          } else if (nt_out) {
            c_qk = prefetch_w<false>(a.w_out, a.wb_out, D / 32, nout, 1, 0, D / 32, sm.slotA);
          }
        }
        xw(a);
      }
      // ================= down projection: XCD x's slice, partial sums over all hidden columns
      {
        if (copy_wave()) vm_wait_le(c_qk);   // down weights landed (the next QKV weights may still fly)
        __syncthreads();
        V16 ews[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          ews[s2] = W8 ? col4(lw.sdown, nod[s2] * 16 + 4 * eq, D, t < 256 && er < M && s2 < nt_od)
                       : as_v(f32x4{1.f, 1.f, 1.f, 1.f});
        f32x4 v[2];
        xgemm<W8, kSc1>(xl + a.o_act, (uint32_t)(64 * (a.F / 8) * 2), a.F / 256, 0, a.F / 256, M, nt_od, 4, sm.slotB,
                  (float*)&sm.slotB[2048], v);
        if (t < 256 && er < M) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 >= nt_od) break;
            const int n = nod[s2] * 16 + 4 * eq;
            const V16 wsv = ews[s2];
            const Rsrc rp = make_rsrc(a.part + (size_t)(8 + me.x) * 64 * D, (uint32_t)(64 * D * 4));
            st16<kSc1>(rp, (uint32_t)((er * D + n) * 4), as_v(as_f4(wsv) * v[s2]));
          }
        }
        if (!copy_wave()) wait_all();
        __syncthreads();
        if (t == 0) flag_st(a.flags + kXFd + me.r * 8 + me.x, la.pe0 + npe);
        // copy waves: the next layer's prefix key tiles (slot B is free after the down GEMM),
        // behind the flag
        if (l + 1 < a.L) {
          __syncthreads();
          issue_tiles(a, l + 1);
        }
      }
      // ================= reduce the down partials + residual; publish the next norm operand ==
      {
        part_wait(a, me, kXFd, 4 * me.x, 8, la.pe0 + npe, sm);
        if (t < 2 * tpr) {
          const int rs = t / tpr, m = 2 * me.r + rs, n = bw * me.x + 4 * (t % tpr);
          const bool ok = m < M;
          const V16 g = col4(site_v(su, 2), n, D, ok);
          const V16 sc = col4(site_v(sn, 0), n, D, ok);
          V16 p[8];
#pragma unroll
          for (int y = 0; y < 8; ++y) {
            const Rsrc rp = make_rsrc(a.part + (size_t)(8 + y) * 64 * D, (uint32_t)(64 * D * 4));
            p[y] = ld16<kSc1>(rp, ok ? (uint32_t)((m * D + n) * 4) : kOob);
          }
          f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int y = 0; y < 8; ++y) sum += as_f4(p[y]);
          f32x4 h = *(f32x4*)&sm.hkeep[rs][4 * (t % tpr)];
          h += as_f4(g) * sum;
          *(f32x4*)&sm.hkeep[rs][4 * (t % tpr)] = h;
          publish(a, me, agb(sn), tpr, rs, m, n, ok, h, as_f4(sc));
        }
        ag_arrive(a, me);
        ++nag;
      }
    }
    // ================= final norm + velocity projection + Euler update (every XCD) ============
    {
      if (copy_wave()) vm_wait_le(0);   // output-projection weights landed
      ag_wait(a, me, la.ag0 + 32u * nag, sm);
      char* ab = agb(2 * a.L);
      load_rinv(a, ab + a.o_agst, sm);
      f32x4 v[2];
      xgemm<false>(ab, (uint32_t)a.o_agst, D / 32, 0, D / 32, M, nt_out, 8, sm.slotA, (float*)sm.slotA, v);
      const int n = me.r * 16 + 4 * eq;
      if (nt_out && t < 256 && er < M && n < a.da) {
        const V16 cv = col4(cvec(2 * a.L), n, a.cout4);
        const V16 bo = col4(a.b_out, n, a.cout4);
        const Rsrc rxx = make_rsrc(xl + a.o_xx, (uint32_t)(M * a.da * 4));
        const V16 xo = ld16<kSc1>(rxx, (uint32_t)((er * a.da + n) * 4));
        const Rsrc rd = make_rsrc(a.dts, (uint32_t)(a.max_steps * 4));
        const float dt = __uint_as_float(ld4<0>(rd, (uint32_t)(k * 4)));
        const f32x4 vel = sm.rinv[er] * v[0] + as_f4(cv) + as_f4(bo);
        if (la.vout) {
          if (me.x == 0) {
            const Rsrc rv = make_rsrc(la.vout, (uint32_t)(M * a.da * 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (n + j < a.da) st4<kSc1>(rv, (uint32_t)((er * a.da + n + j) * 4), __float_as_uint(vel[j]));
          }
        } else {
          const f32x4 xn = as_f4(xo) + dt * vel;
          const Rsrc ro = make_rsrc(la.xout, (uint32_t)(M * a.da * 4));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n + j < a.da) {
              st4<0>(rxx, (uint32_t)((er * a.da + n + j) * 4), __float_as_uint(xn[j]));
              if (me.x == 0) st4<kSc1>(ro, (uint32_t)((er * a.da + n + j) * 4), __float_as_uint(xn[j]));
            }
        }
      }
      xb(a);   // this XCD's x is advanced before its next in-projection reads it
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy outlives the kernel
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
void xloop_counts(int L, int steps, uint32_t* nxb, uint32_t* nag, uint32_t* npe) {
  *nxb = 1u + (uint32_t)steps * (4u * L + 1u);
  *nag = (uint32_t)steps * (2u * L + 1u);
  *npe = (uint32_t)steps * L;
}

static long rup(long x, long m) { return (x + m - 1) / m * m; }

XLayout xloop_layout(int B, int H, int D, int F, int da, int npairs) {
  XLayout r;
  r.Hp = (int)rup(H, 32);
  long off = 0;
  auto put = [&](long bytes) { const long o = off; off += rup(bytes > 0 ? bytes : 1, 4096); return o; };
  r.o_xx = put(64L * da * 4);
  r.o_q = put((long)B * 64 * 256 * 2);
  r.o_sk = put((long)B * r.Hp * 256 * 2);
  r.o_svt = put((long)B * 256 * r.Hp * 2);
  r.o_ap = put((long)npairs * 64 * 256 * 4);
  r.o_ml = put((long)npairs * 64 * 8);
  r.o_ax = put(64L * 256 * 2);
  r.o_act = put(64L * (F / 8) * 2);
  r.xl_stride = off;
  r.o_agst = 64L * D * 2;
  r.ag_site = rup(r.o_agst + 64L * 8 * 4, 4096);
  return r;
}

const char* xloop_check(const XShape& s, int num_cus) {
  if (!s.bf16) return "bf16 only";
  if (s.dh != 256) return "head_dim 256 only";
  if (num_cus != 256) return "a device of 256 CUs (8 XCDs of 32) only";
  if (s.nq < 1 || s.nq > 8) return "1 to 8 query heads (one per XCD)";
  if (s.B * s.H < 1 || s.B * s.H > 64) return "batch x horizon must be at most 64 rows";
  if (s.B > kXMaxReq) return "too many requests";
  if (s.D != 512 && s.D != 1024) return "hidden 512 or 1024";
  if (s.F % 512 != 0 || s.F > 4096) return "mlp_dim a multiple of 512, at most 4096";
  if (s.da % 4 != 0 || s.da > 32) return "action_dim a multiple of 4, at most 32";
  if (s.L < 1 || s.L > kXMaxLayers) return "1 to 64 layers";
  if (s.npairs > kXMaxPairs) return "more than 32 key-tile pairs per head (64 key tiles over the requests)";
  return nullptr;
}

hipError_t xloop_launch(const XLoopArgs* a_dev, const XLaunch& la, bool w8, hipStream_t s) {
  const XLoopArgs* p = a_dev;
  XLaunch l2 = la;
  void* args[] = {&p, &l2};
  if (w8) return hipLaunchCooperativeKernel((const void*)k_xloop<true>, dim3(256), dim3(kT), args, 0, s);
  return hipLaunchCooperativeKernel((const void*)k_xloop<false>, dim3(256), dim3(kT), args, 0, s);
}

}  // namespace fm
