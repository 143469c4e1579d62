// Internal launch interfaces of the denoise-loop kernels (not part of the public C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

enum ElemType { ET_F32 = 0, ET_BF16 = 1 };
enum EpiKind { EPI_STORE = 0, EPI_GELU_MUL = 1, EPI_QKV = 2, EPI_RESID = 3, EPI_EULER = 4, EPI_VT = 5 };
enum Act { ACT_NONE = 0, ACT_SILU = 1, ACT_GELU = 2 };
enum NormKind { NORM_NONE = 0, NORM_RMS = 1, NORM_LN = 2 };

// Columns per partial row-statistic slot written by the residual epilogue and the
// in-projection, and read by the consumer GEMMs of the next modulated norm. Statistics
// are (mean, M2) float2 pairs laid out [row][slot]; hidden / kStatCols slots per row.
constexpr int kStatCols = 32;
constexpr int kMaxStatSlots = 64;   // hidden <= 2048

// C[M x N] = A[M x K] * W^T, W stored fragment-major (see swizzle_weight).
//
// Modulated norms are folded around the GEMM: with u = (h - mu) rinv (1 + s) + t,
//   u W^T = rinv (hs W^T - mu d) + c,   hs = h (1 + s),  d = (1 + s) W^T,  c = t W^T,
// so the producer of h also writes hs (rounded to T) and per-slot row statistics, the
// schedule precomputes c and d per step, and the consumer's epilogue applies rinv, mu, c, d.
struct GemmArgs {
  int M, N, K;
  // A operand: a row-major T matrix; row r is read from row (r/row_group)*row_gstride +
  // row_off + r%row_group
  const void* A; long lda;
  int row_group, row_gstride, row_off;
  // consumer side of a modulated norm (norm != NORM_NONE): per-row (mu, rinv) merged from
  // stats[row * stats_ld + slot] of the A rows (nparts slots of kStatCols columns);
  // y = rinv (acc - mu d[n]) + c[n] (d only for LayerNorm)
  int norm;
  const float2* stats; int nparts; long stats_ld;
  const float* cvec; const float* dvec;
  float eps;
  // B operand: fragment-major weights of [Npad x K]
  const void* W;
  // split-K (tiled kernel only)
  int splits, k_split;
  float* ws; unsigned* counters;
  // epilogue
  int epi;
  void* out; long ldo; const float* bias; int act; int out_f32;
  // residual producer: h += gate * y; hs = T(h (1 + hscale)); (mean, M2) of h per
  // kStatCols columns at stats_out[row * stats_out_ld + n / kStatCols]
  float* h; long ldh_out; const float* gate; void* hs; const float* hscale; float2* stats_out; long stats_out_ld;
  int q_cols, kv_cols, tq, kv_off, rope, half_dh; const float2* rope_cs;   // rope_cs [M rows][half_dh]: each row's position
  void* kdst; long k_bs, k_rs; void* vdst; long v_bs, v_ds;
  float* x; float dt; float* vout;
  int vt_group; long vt_bs, vt_ds;
  // Device buffers of at least kVecPad zeros / ones that the launcher substitutes for
  // absent optional vectors (kernels never test pointers; an absent gate reads ones).
  const float* zeros; const float* ones;
  // byte extents of A, W and the split-K workspace, set by the launcher (each < 2^31: reads
  // at or past them return zeros)
  uint32_t a_bytes, w_bytes, ws_bytes;
  // launch shape chosen by the planner
  int kind;          // GEMM_SKINNY / GEMM_TILED
  int cfg;           // tile configuration of that kind
  int cpw;           // skinny: k-chunks per wave
  int kw;            // skinny: waves per workgroup (4 / 8)
  // EPI_STORE / EPI_VT column planes: output column n is column n % col_group of plane
  // n / col_group, the planes col_gstride elements apart (col_group 0: one plane). Kept last,
  // so that the fields above keep their offsets in the kernel arguments.
  int col_group; long col_gstride;
  // Optional FP8 E4M3 copy of the weights (codes fragment-major as swizzle_fp8, with the
  // matrix's per-row power-of-two scales by output column, padded to N rounded up to 4). The
  // planner sets fp8 when the skinny kernel then streams the codes instead of W (bf16, K a
  // multiple of 64); the sums are scaled per column before the epilogue.
  const void* w8; const float* wscale; int fp8;
  // Weight-streaming kernel over more than 64 rows: rgroups groups of 64 rows, each a workgroup
  // of its own per column tile and split (0 or 1: one group, M <= 64).
  int rgroups;
};
constexpr long kVecPad = 1L << 18;   // floats in the zeros / ones buffers
// Split-K arrival counters (GemmArgs::counters): one per output tile.
constexpr int kGemmCounters = 1 << 16;

enum GemmKind { GEMM_SKINNY = 0, GEMM_TILED = 1, GEMM_BIG = 2 };
enum GemmCfg { GEMM_64x64 = 0, GEMM_128x128 = 1, GEMM_32x64 = 2 };
enum SkinnyCfg { SK_N16 = 0, SK_N32 = 1 };   // 16 * (cfg + 1) output columns per workgroup

// Plan kernel, tile shape and split-K for an M x N x K problem.
void gemm_plan(GemmArgs& a, int elem, int num_cus);
size_t gemm_ws_bytes(const GemmArgs& a);        // split-K partial workspace bytes
int gemm_num_tiles(const GemmArgs& a);
hipError_t gemm_launch(const GemmArgs& a, int elem, hipStream_t s);

// Attention (vla.cpp Eq. (2); its additive mask as the visibility fields below) over groups of
// query rows sharing one K/V head.
struct AttnArgs {
  const void* q; long q_bs, q_rs;             // q[b*q_bs + t*q_rs + n*dh + d]
  const void* k; long k_bs, k_rs, k_hs;       // k[b*k_bs + g*k_hs + j*k_rs + d]
  const void* vt; long v_bs, v_hs, v_ds;      // v transposed: vt[b*v_bs + g*v_hs + d*v_ds + vt_slot(j)]
  long k_len, v_len;                          // elements readable from k / vt (reads past them give 0)
  void* o; long o_bs, o_rs;                   // o[b*o_bs + t*o_rs + n*dh + d]
  int B, Tq, n_heads, heads_per_kv, n_keys, dh;
  float scale_log2;                            // log2(e) / sqrt(dh)
  int splits, keys_per_split;
  float* ws;                                   // split partials (attn_ws_bytes), merged by a second kernel
  int cfg;
  // Per-request key visibility (the additive mask of Eq. (2): 0 or -inf), null = every key:
  //  seg_len: request b sees keys [0, seg_len[b]) of its leading segment and every key in
  //    [seg_end, n_keys) (a compact prefix of its own length, then its chunk's keys);
  //  kmask: request b sees key j when bit j % 32 of kmask[b * km_bs + j / 32] is set.
  // Kept last: placed between the fields above they moved those fields' offsets, and the
  // attention kernel's argument loads then ran measurably slower (62 -> 66 us at 64 requests).
  const int* seg_len; int seg_end;
  const uint32_t* kmask; long km_bs;
};
void attn_plan(AttnArgs& a, int elem, int num_cus);
size_t attn_ws_bytes(const AttnArgs& a);
int attn_num_items(const AttnArgs& a);
hipError_t attn_launch(const AttnArgs& a, int elem, hipStream_t s);

// Fragment-major weight layout: dst holds ceil(N/16) x (K/KC) fragments of 64 x 16 bytes.
// src is [N x K] row-major; rows listed by src_rows (device, length N; -1 = zero row) or identity.
hipError_t swizzle_weight(void* dst, const void* src, const int* src_rows, int N, int K, long ld_src,
                          int elem, hipStream_t s);
size_t swizzled_bytes(int N, int K, int elem);

// h rows of the in-projection, with per-slot row statistics for the first norm.
struct InProjArgs {
  const float* zeros;                         // kVecPad zeros, read for absent tb / hscale / state_tok
  const float* x; int da;                     // x [B*Ha x da] fp32
  const void* w; const float* b;              // w [D x da] (T, row-major), bias fp32 [D]
  const float* tb;                            // per-step time bias fp32 [D] or null
  const float* state_tok;                     // [B*st x D] fp32 or null
  int B, Ha, st, D;                           // rows per request = st + Ha
  float* h; float2* stats; long stats_ld;     // stats[row * stats_ld + slot], kStatCols columns per slot
  void* hs; const float* hscale;              // hs = T(h (1 + hscale)) (hscale may be null)
};
hipError_t inproj_launch(const InProjArgs& a, int elem, hipStream_t s);

hipError_t convert_to_f32(float* dst, const void* src, long n, int elem, hipStream_t s);
hipError_t convert_from_f32(void* dst, const float* src, long n, int elem, hipStream_t s);
// Prefix K into the pool with RoPE pair interleave (d' = 2j <- j, 2j+1 <- j + dh/2) when rope.
hipError_t prefix_k_copy(void* pool, long pool_bs, const void* src, int B, int P, int dh, int rope,
                         int elem, hipStream_t s);
// Prefix V into the pool transposed: pool[b*pool_bs + d*cap + vt_slot(j)] = src[(b*P + j)*dh + d].
hipError_t prefix_v_copy_t(void* pool, long pool_bs, int cap, const void* src, int B, int P, int dh,
                           int elem, hipStream_t s);
hipError_t fill_f32(float* dst, float v, long n, hipStream_t s);
// out[b] = the XCC id workgroup b of an n-workgroup launch runs on (n <= 65536)
hipError_t xcc_probe(uint32_t* out, int n, hipStream_t s);
// FP8 E4M3 weights, one power-of-two scale per row: codes [N x K] bytes, scale [N], and the
// dequantized bf16 matrix deq [N x K] (exact). src bf16 rows of stride ld; K even.
hipError_t quantize_fp8_rows(const void* src, long ld, int N, int K, uint8_t* codes, float* scale, void* deq, hipStream_t s);
// FP8 codes fragment-major (16 rows x 64 k per 1 KB fragment; K a multiple of 64), rows as swizzle_weight.
hipError_t swizzle_fp8(void* dst, const uint8_t* codes, const int* rows, int N, int K, hipStream_t s);
size_t swizzled_fp8_bytes(int N, int K);
// dst[i] = src[rows[i]] (or src[i]) for i < N, 0 for N <= i < Npad
hipError_t gather_f32(float* dst, const float* src, const int* rows, int N, int Npad, hipStream_t s);
// model-space chunk -> robot units, first hr steps and dr dims (kind 0 / 1 as fm.h)
hipError_t unnormalize_launch(const float* x, float* out, const float* q01, const float* q99, int B, int H, int da,
                              int hr, int dr, int kind, hipStream_t s);
// dst[r*dld + c] = T(src[r*sld + c] + add) for r < rows, c < cols.
hipError_t rows_from_f32(void* dst, long dld, const float* src, long sld, int rows, int cols, float add, int elem,
                         hipStream_t s);

}  // namespace fm
