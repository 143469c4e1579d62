// Internal interface of the persistent denoise-loop kernel (fm_persist.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

constexpr int kMaxLayers = 64;
constexpr int kMaxSA = 16;         // attention key splits per row tile
constexpr int kMaxGrid = 256;        // one workgroup per CU; the barrier polls 256 flags at once
constexpr int kMaxSplitItems = 512;  // split-K GEMM items per phase
constexpr int kMaxAttnItems = 256;   // attention items (row tile x key split) per layer
constexpr int kMaxRowTiles = 64;     // attention row tiles (64 folded query rows) per layer
// flag words: [0, 256) arrival epochs, release epoch, error word, split-K item flags,
// attention split flags [row tile][split]
constexpr int kFlagRelease = 256;
constexpr int kFlagErr = 260;
constexpr int kFlagSplit = 512;
constexpr int kFlagAttn = kFlagSplit + kMaxSplitItems;
constexpr int kFlagWords = kFlagAttn + kMaxRowTiles * kMaxSA;

// Fragment-major weights of one layer.
// With FP8 weights the four matrices hold codes and s* their per-row scales (padded to 4
// floats); with bf16 weights the s* are null.
struct LayerW {
  const void* qkv; const void* o; const void* gu; const void* down;
  const float* sqkv; const float* so; const float* sgu; const float* sdown;
};

// Shapes that decide whether the loop kernel applies.
struct LoopShape {
  int dtype_bf16, B, H, M, D, nq, dh, F, da, L, P;
  int qd;   // nq * dh
};

struct LoopArgs {
  int B, H, M, D, nq, dh, F, da, L, P, cap;
  int qd, nqkv, Hp, S;
  long csum;
  int cq4, cg4, cout4;
  float eps, scale_log2;
  int rope;
  int RT, TP, TS, SA;            // attention: row tiles per request, prefix / suffix key tiles, splits
  int max_steps;
  const float* dts;              // [max_steps] tau[k+1] - tau[k]
  const void* w_in; const float* b_in;
  const void* w_out; const float* b_out;
  const LayerW* lw;               // [L] per-layer weights (device table)
  uint32_t wb_qkv, wb_o, wb_gu, wb_down, wb_out;
  const float* table;            // [steps][S][3D]
  const float* cbuf;             // [steps][csum]
  const float2* rope_cs;         // [B][H][dh / 2]: cos / sin at each request's positions P_b + i
  float* x; float* h;
  const __bf16* pool; long plane;   // elements per pool plane
  char* rot; long rot_step, rot_layer;
  long o_hs, o_st, o_q, o_sk, o_svt, o_ao, o_hsu, o_stu, o_act;
  float* ws_attn; float* ws_attn_ml; float* ws_split;
  uint32_t* flags;
  const int* plens;              // [B] compact prefix length P_b <= P of each request (kept last)
};

// Per-launch arguments: first step, step count, first barrier epoch, and the velocity
// output of a single-step launch (null: Euler-update x).
struct LaunchArgs {
  int k0, nsteps;
  uint32_t e0;
  float* vout;
};

// nullptr when the loop kernel supports the shape on a device with num_cus CUs, else why not.
const char* loop_check(const LoopShape& s, int num_cus);
// grid barriers one launch of `steps` Euler steps performs
int loop_barriers(int L, int steps);
// a: the loop description in DEVICE memory (read by the kernel through a pointer)
// w8: the LayerW matrices are FP8 codes (k_loop<true>)
hipError_t loop_launch(const LoopArgs* a_dev, const LaunchArgs& la, int grid, bool w8, hipStream_t s);

}  // namespace fm
