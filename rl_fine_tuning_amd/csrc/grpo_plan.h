// Host-side validation and workspace planning shared by the entry points.
// Pure C++: no HIP headers, so the checks run (and are tested) without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "grpo.h"

namespace grpo {

// MFMA workgroup tiles.  fp32 inputs: 256 x 256 (vocabulary or hidden x tokens).  bf16
// inputs: 256 rows of the first operand x 256 tokens, with the tokens' operand in a
// fragment-major copy (16-element k steps, 256-row tiles).
constexpr int kTile = 256;
constexpr int kTileA16 = 256;
constexpr int kTileB16 = 256;
// MI355X compute units; sizes the vocabulary split of the dH GEMM for small chunks.
constexpr int kNumCUs = 256;
constexpr int kMaxKSplit = 8;
constexpr size_t kAlign = 256;
// Banded W^T for the dH GEMM: used for chunks of at least this many tokens (below, the
// transposes of W in every backward pass cost more than the faster GEMM saves) and bands of
// at least this many k steps of 16 vocabulary entries.
constexpr int64_t kBandMinRows = 2048;
constexpr int64_t kBandMinKs = 64;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// K-step of the GEMM main loop: one 128-byte LDS row per operand row.
inline int k_step(int32_t dtype) { return dtype == GRPO_BF16 ? 64 : 32; }
inline int elem_size(int32_t dtype) { return dtype == GRPO_BF16 ? 2 : 4; }

struct Plan {
  int64_t T = 0, D = 0, V = 0, C = 0, nchunks = 0, S = 0;
  int32_t dtype = 0;
  int esize = 0, bk = 0;
  int64_t ntiles_v = 0;   // vocabulary tiles = (max, sum-exp) partials per token
  int64_t ldp = 0;        // fp32: row stride (elements) of the chunk probability matrix
  int64_t rows_pad = 0;   // bf16: chunk rows rounded up to the 256-row tile
  int64_t ks_d = 0;       // bf16: k steps of 16 over D (fragment-major hidden states)
  int64_t ks_v = 0;       // bf16: k steps of 16 over V (fragment-major probabilities)
  bool use_wt = false;    // bf16: the dH GEMM reads a fragment-major W^T from the workspace
  bool use_wf = false;    // bf16: the logits GEMMs read a fragment-major W from the workspace
  int64_t bwd_rows = 0;   // tokens per backward slice (bf16: a multiple of 256; >= C when unsliced)
  int64_t qt_tiles = 0;   // bf16 with dW: vocabulary tiles per band of the dW GEMM's transposed operand
  bool dh32 = false;      // bf16 backward writing fp32 dH: the probabilities as bf16 hi + lo pairs
  int64_t ks_q = 0;       // bf16: k steps per row of the probability buffer (ks_v, or 2 ks_lo with dh32)
  int64_t ks_lo = 0;      // bf16 with dh32: first k step of the lo half (ks_v rounded up to even)
  int64_t wt_band_ks = 0; // bf16 without room for the whole W^T copy: k steps (vocabulary / 16) per band
                          // of W^T transposed in each backward pass (even); 0: no bands
  int64_t wt_bands = 0;   // number of such bands (>= 2 when used)
  bool backward = false;
  bool host_h = false;    // backward from hidden states in pinned host memory: chunks staged in the workspace
  size_t off_Hs = 0;      // host_h: two staging buffers of one chunk's rows of H
  size_t hs_bytes = 0;    // host_h: bytes of one staging buffer
  size_t off_zy = 0, off_lse = 0, off_pm = 0, off_ps = 0;
  size_t off_g = 0, off_wl = 0, off_seq = 0, off_cu = 0, off_cnt = 0, off_wseq = 0;
  size_t off_P = 0, off_part = 0, off_Hf = 0, off_WT = 0, off_Wf = 0, off_Qt = 0, off_WTb = 0;
  size_t total = 0;
};

// Logits from the raw lm_head products x = H[t] . W[v]: z = zscale * v with v = x, or with a
// softcap v = tanh(cap_in * x); dz/dx = dscale, or dscale * (1 - v^2) with the softcap.
struct LogitMap {
  float zscale;
  float dscale;
  float cap_in;  // 0: no softcap
};
LogitMap make_logit_map(const grpo_shape* s);  // s already validated

// Vocabulary split of the dH GEMM for a backward slice of `rows` tokens.
int dh_ksplit(int64_t rows, int64_t D, int64_t V, int32_t dtype);

grpo_status validate_shape(const grpo_shape* s);
grpo_status validate_loss_params(const grpo_loss_params* p);
grpo_status validate_cu(const int32_t* cu, int64_t S, int64_t T);
grpo_status make_plan(const grpo_shape* s, int64_t S, bool backward, Plan* out, bool dW = false, bool host_h = false);
// with_backward of grpo_workspace_bytes / grpo_plan_info: 0, 1, 2, and 1 or 2 plus GRPO_WS_HOST_H
bool decode_ws_mode(int with_backward, bool* backward, bool* dW, bool* host_h);
int dh_ksplit(int64_t chunk_rows, int64_t D, int64_t V, int32_t dtype);
bool aligned16(const void* p);

}  // namespace grpo
