// Internal interface of the XCD-parallel denoise-loop kernel (fm_xloop.hip): every Euler step
// of a chunk of at most 64 action rows in one cooperative launch of one workgroup per CU, the
// expert's layers split across the 8 XCDs the way tensor parallelism splits them across
// devices (query heads, MLP columns and the rows of the output projections), with the two
// reductions per layer exchanged between XCDs and every other dependency kept inside one XCD.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

constexpr int kXMaxPairs = 32;   // attention key-tile pairs of one head, over all requests: one per CU of an XCD
constexpr int kXMaxReq = 64;
constexpr int kXMaxLayers = 64;

// Flag words (uint32), each group on its own cache lines:
//   XCD barrier counters at kXBar + 32 x (XCD-local: updated and read by L2 atomics),
//   norm-operand counters at kXAg + 32 c (device scope: XCD c's share of a norm operand is out),
//   O / down partial flags [rank][xcd] (device scope), the fault word, the (XCD, rank) slots, and
//   per-XCD release words (XCD-local): rank 0 of an XCD alone polls the device-scope words of a
//   cross-XCD wait and then releases its XCD through these.
constexpr int kXBar = 0;
constexpr int kXAg = 256;
constexpr int kXFo = 512;
constexpr int kXFd = 768;
constexpr int kXErr = 1024;
constexpr int kXSlot = 1056;
constexpr int kXRelAg = 1312;    // at + 32 x: the norm-operand wait of XCD x is satisfied up to this value
constexpr int kXRelO = 1568;     // at + 32 x: the O partial-sum wait of XCD x
constexpr int kXRelD = 1824;     // at + 32 x: the down partial-sum wait of XCD x (the O and down
                                 // waits of a layer share one target value, so not one word)
constexpr int kXFlagWords = 2080;
// fault word values: 1 an XCD barrier, 2 a norm-operand wait, 3 an O / down partial wait
// expired; 4 two workgroups took one (XCD, rank) slot (the dispatch was not round-robin)
constexpr uint32_t kXFaultSlot = 4;

// Fragment-major weights of one layer (FP8: codes, and per-row scales padded to 4 floats).
struct XLayerW {
  const void* qkv; const void* o; const void* gu; const void* down;
  const float* sqkv; const float* so; const float* sgu; const float* sdown;
};

// A pair of key tiles of the attention of one head: request b, tiles j and j + 1 of its key list
// (its ceil(P_b / 32) prefix tiles, then the chunk's ceil(H / 32) tiles); j + 1 may be past the
// list. One CU of each XCD takes one pair, a half of the workgroup per tile.
struct XPair { int b, j; };

struct XLoopArgs {
  int B, H, M, D, nq, F, da, L, P, cap, Hp, S;
  long csum;
  int cq4, cg4, cout4;
  float eps, scale_log2;
  int rope, max_steps;
  int npairs;                       // attention key-tile pairs of one head, all requests
  XPair pair[kXMaxPairs];
  int poff[kXMaxReq + 1];           // request b's pairs: [poff[b], poff[b + 1])
  int plen[kXMaxReq];               // compact prefix length P_b of each request
  const float* dts;                 // [max_steps] tau[k + 1] - tau[k]
  const void* w_in; const float* b_in; const void* w_out; const float* b_out;
  const XLayerW* lw;                // [L]
  uint32_t wb_qkv, wb_o, wb_gu, wb_down, wb_out;
  const float* table;               // [steps][S][3D]
  const float* cbuf;                // [steps][csum]
  const float2* rope_cs;            // [B][H][128]: cos / sin at request b's positions P_b + i
  const __bf16* pool; long plane;
  // XCD-local buffers: region of XCD x at xl + x * xl_stride
  char* xl; long xl_stride;
  long o_xx, o_q, o_sk, o_svt, o_ap, o_ml, o_ax, o_act;
  // cross-XCD: O / down partial sums [2][8][64][D] fp32, and the norm operands of every
  // (step, site): bf16 h (1 + scale) [64][D] fragment-major, then row sums of squares [64][8]
  float* part;
  char* ag; long ag_site, ag_step, o_agst;
  uint32_t* flags;
};

// Per launch: first step and step count; counter bases (the values the XCD barrier counters,
// the norm-operand counters and the partial flags hold at launch start); the chunk read at the
// first step (xin) and the chunk written after every step (xout; may equal xin), or the
// velocity output of a single-step launch (vout: x is then not advanced).
struct XLaunch {
  int k0, nsteps;
  uint32_t xb0, ag0, pe0;
  const float* xin; float* xout; float* vout;
};

struct XShape {
  int bf16, B, H, D, nq, dh, F, da, L;
  int npairs;   // attention key-tile pairs of one head over the bound requests
};

// nullptr when the kernel serves the shape on a device with num_cus CUs, else why not.
const char* xloop_check(const XShape& s, int num_cus);
// XCD barriers, norm-operand exchanges and partial exchanges of one launch
void xloop_counts(int L, int steps, uint32_t* nxb, uint32_t* nag, uint32_t* npe);
// Buffer layout for a binding: per-XCD region bytes and offsets, norm-operand sizes.
struct XLayout { long o_xx, o_q, o_sk, o_svt, o_ap, o_ml, o_ax, o_act, xl_stride; long ag_site, o_agst; int Hp; };
XLayout xloop_layout(int B, int H, int D, int F, int da, int npairs);
hipError_t xloop_launch(const XLoopArgs* a_dev, const XLaunch& la, bool w8, hipStream_t s);

}  // namespace fm
