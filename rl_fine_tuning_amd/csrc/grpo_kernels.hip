// gfx950 (MI355X) kernels and C-ABI entry points of the chunked GRPO path.
//
// What is computed follows the Unsloth pages:
//  * "Reinforcement Learning GRPO mit 7x laengerem Kontext" (Unsloth docs), the call of
//    chunked_hidden_states_selective_log_softmax: logits = hidden states x lm_head over
//    a chunk of the flattened token stream, upcast to fp32, divided by the temperature,
//    log-softmaxed and gathered at the target id; section "Auslagern von Aktivierungen
//    fuer Log-Softmax": nothing but log-probabilities is kept from the forward and the
//    backward recomputes the chunk's logits.
//  * "Unsloth internals", section "The relationship to TRL": group-relative advantages,
//    clipped surrogate, KL-to-reference term; "You can now train reasoning models with
//    5GB VRAM thanks to Unsloth", section "Under the Hood": reverse KL, ratio
//    exp(logp - old_logp) times the sequence's advantage.
//
// How it is laid out on the chip (not from the pages):
//  * One GEMM kernel template, 256 threads (4 waves of 64), one 256 x 256 output tile
//    per workgroup, v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x2f32 for fp32 inputs),
//    each wave a 128 x 128 sub-tile held as 4 x 4 accumulator blocks in AGPRs.  K is
//    staged through LDS in 128-byte rows (64 bf16 / 32 fp32), double buffered, with an
//    XOR swizzle of the 16-byte chunks so that operand reads and staging writes avoid
//    bank conflicts.
//  * The logits GEMMs put the vocabulary on the MFMA row axis and tokens on the column
//    axis, so a lane holds 64 vocabulary entries of 4 tokens: the per-token max and
//    sum-exp need only in-lane work plus one cross-lane step, and probability rows are
//    written as 4-element vectors.
//  * The dH GEMM computes dH^T tiles (hidden x tokens) with K = vocabulary.  W [V, D] is
//    read as its transpose by loading 8 x 8 blocks and transposing them in registers on
//    the way into LDS, so no transposed copy of W is ever stored.
//  * Workgroups are dispatched round-robin over the 8 XCDs; the tile map gives each XCD
//    a contiguous share of one tile axis and walks the other in small groups, so the
//    workgroups that run together on one XCD share operand tiles in its L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "grpo.h"
#include "grpo_plan.h"

// Workspace of grpo_loss_fwd_bwd_static (for callers that cannot allocate): one copy per
// device, held from the library's load until the process ends.  Every call on a device
// uses the same bytes; each call writes every byte it reads, so nothing needs clearing.
constexpr size_t kStaticScratchBytes = size_t(256) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

struct grpo_timer {
  int32_t capacity = 0;
  int32_t used = 0;
  int64_t dropped = 0;
  std::vector<hipEvent_t> start, stop;
  std::vector<int32_t> kid;
};

// Host offload of the hidden states: a copy stream beside the caller's and the events that
// order the two.
struct grpo_offload {
  hipStream_t copy = nullptr;
  hipEvent_t ev_in = nullptr;     // recorded on the call's stream when the call starts
  hipEvent_t ev_done = nullptr;   // forward: the copy of H to the host has finished
  hipEvent_t ev_ready[2] = {};    // backward: staging buffer b holds its chunk
  hipEvent_t ev_free[2] = {};     // backward: the chunk in staging buffer b has been used
};

namespace grpo {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;                   // one LDS tile row: 8 chunks of 16 bytes
constexpr int kTileBytes = kTile * kRowBytes;    // one operand, one stage: 32 KB
constexpr float kLog2e = 1.4426950408889634f;

// KIND_DH reads W for the dH GEMM transposed on the fly; KIND_DHT (bf16) reads a
// fragment-major copy of W^T with direct-to-LDS loads.
// KIND_LSES (bf16): the LSE epilogue that also keeps the chunk's logits, as d = z - (tile
// max) in fp16, in the probabilities buffer (the variant without the recompute GEMM).
// KIND_DW (bf16): dW += Gx^T H_c over one vocabulary band, A = the band of Q^T in fragment-major
// order (qt_band_kernel), read by direct-to-LDS loads like the copy of W.
enum Kind { KIND_LSE = 0, KIND_PROBS = 1, KIND_DH = 2, KIND_DHT = 3, KIND_LSES = 4, KIND_DW = 5 };

// Byte offset of 16-byte chunk c of row r inside a [256 rows x 8 chunks] LDS tile.
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kRowBytes + ((c ^ ((r & 7) ^ ((r >> 3) & 7))) << 4);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// (a vector conversion: one packed convert instruction for the pair)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t v = {a, b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Two floats as fp16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float f16_lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }

// The low (hi = false) or high 16-bit halves of x and y as one word, x's half in the low
// 16 bits: v_perm_b32 picks bytes of the 64-bit pair whose bytes 0-3 are its second
// operand (x here) and bytes 4-7 its first (y).
__device__ __forceinline__ uint32_t halves(uint32_t x, uint32_t y, bool hi) {
  return __builtin_amdgcn_perm(y, x, hi ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// LogitMap (grpo_plan.h): temperature tau, scale s = multiply / divide, softcap c.  Without
// a cap zscale = dscale = s / tau; with it zscale = c / tau, dscale = s / tau, cap_in = s / c.

// tanh(a) from its definition (e^{2a} - 1) / (e^{2a} + 1) = 1 - 2 / (e^{2a} + 1), with the
// Taylor series a - a^3 / 3 for |a| < 2^-6, where the subtraction would cancel; saturates
// to +-1 for large |a|.
__device__ __forceinline__ float tanh_fast(float a) {
  const float e = __builtin_amdgcn_exp2f(2.0f * kLog2e * a);
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  const float s = a * fmaf(-a * a, 1.0f / 3.0f, 1.0f);  // |a| < 2^-6: keeps tanh's relative precision
  // Both forms are computed and one is picked by a byte permute (selector bytes 4..7 take the
  // first operand, 0..3 the second), so the choice stays a per-lane select, never a branch.
  const uint32_t sel = fabsf(a) < 0.015625f ? 0x07060504u : 0x03020100u;
  return __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(s), __float_as_uint(t), sel));
}

struct GemmArgs {
  const void* a;      // LSE / PROBS: W [V, D] or its fragment-major copy.  DH: W [V, D], read
                      // transposed.  DHT: the fragment-major copy of W^T.  DW: (-c H)^T, fragment-major
  const void* b;      // LSE / PROBS: hidden-state chunk [rows, D].  DH: probabilities [rows, ldp].
                      // DW: the band of Q^T, fragment-major
  int64_t lda, ldb;   // row strides (elements)
  int a_rows;         // rows of the MFMA A operand: V (LSE / PROBS) or D (DH, DW)
  int b_rows;         // tokens in the chunk (DW: rows of the band)
  int K;              // reduction length: D (LSE / PROBS), V (DH) or the slice's tokens (DW)
  int k_len;          // DH: vocabulary entries per split; otherwise K
  int tiles_a_base;   // A tiles before the split factor
  int tiles_a, tiles_b;
  int xcd_a;          // XCD grid: tiles_a in xcd_a ranges, tiles_b in 8 / xcd_a (xcd_a = 1, 2, 4, 8)
  int group_b;        // B tiles walked together
  LogitMap lm;
  // LSE outputs: [tiles_a][b_rows]
  float* pm;
  float* ps;
  // PROBS
  const float* lse;   // [b_rows], chunk-local
  void* p;            // [b_rows, ldp]
  int64_t ldp;
  int V;
  // DH
  const float* g;         // [b_rows]
  const float* zy;        // [b_rows]: target logits (the softcap's W[y] factor)
  float* zy_out;          // LSE / LSES (bf16): [b_rows] target logits captured from the tile
  float* dw;              // DW: [V, D] fp32, offset to the band's first vocabulary row
  int accumulate;         // DW: add to dw (later chunks) instead of overwriting it; DHT with part_out:
                          // add to the partials (the later bands of a banded W^T)
  const int32_t* targets; // [b_rows]
  void* dh;               // [b_rows, D] (ksplit == 1)
  float* part;            // [ksplit][b_rows][D] (ksplit > 1, or part_out)
  int part_out;           // DHT: write the fp32 partials even with ksplit == 1 (banded W^T)
  int k_base;             // DHT: first k of this launch's reduction (a band's first vocabulary entry)
  int a_koff;             // bf16 DHT: k steps subtracted from k / 16 to index the A copy (a band's start)
  int D;
  int ksplit;
  int dh_f32;         // DH / DHT unsplit: dH is written as fp32
  int lo_ks;          // PROBS: also write the lo halves from this k step (0: none)
  int a_ks;           // bf16 DHT: k steps of the A copy when they differ from b_ks (0: same)
  int a_wrap;         // DH / DHT over hi + lo probabilities: A's k step wraps to 0 here (0: none)
  int b_ks;           // bf16: k steps (ceil(K / 16)) of the fragment-major B copy (and A copy)
  int a_frag;         // bf16 LSE / PROBS / LSES: A is the fragment-major copy of W
  int p_ks;           // bf16 PROBS / LSES: k steps per row of the fragment-major probabilities
  int v_ks;           // bf16 PROBS / LSES: k steps written (the vocabulary's, even with hi + lo halves)
};

// The backward's logit gradient Gx[t, v] = dL/dx[t, v] = -c_t Q[t, v] with
// Q = P' - onehot(y_t) wyf_t: P' the probabilities (times 1 - v^2 with a softcap), wyf_t
// the softcap factor at the target (1 - v_y^2, else 1) and c_t = g_t * dscale.  The buffer
// holds Q (the target entry rewritten exactly in fp32 by onehot_fix_kernel); -c_t is
// applied per token by the dH epilogue (and to the tokens' operand of dW).  A token with
// g_t = 0 or a target outside [0, V) gets c_t = 0.
struct TokGrad {
  float c, wyf;
  int y;
  bool live;
};
__device__ __forceinline__ TokGrad tok_grad(const float* g, const int32_t* targets, const float* zy, int V,
                                            const LogitMap& lm, int tok, bool ok) {
  TokGrad r;
  const float gt = ok ? g[tok] : 0.0f;
  r.y = ok ? targets[tok] : -1;
  r.live = gt != 0.0f && r.y >= 0 && r.y < V;
  r.c = r.live ? gt * lm.dscale : 0.0f;
  const float ty = (r.live && lm.cap_in > 0.0f) ? zy[tok] / lm.zscale : 0.0f;
  r.wyf = 1.0f - ty * ty;
  return r;
}

// Tile of this workgroup.  Workgroup i runs on XCD i % 8; each XCD owns a contiguous
// share of one tile axis and walks the other axis group_b tiles at a time.
__device__ __forceinline__ bool map_tile(const GemmArgs& g, int& ta, int& tb) {
  const int bid = blockIdx.x;
  const int xcd = bid & 7;  // workgroups go to the 8 XCDs in turn
  const int local = bid >> 3;
  const int xb_parts = 8 / g.xcd_a;
  const int xa = xcd % g.xcd_a, xb = xcd / g.xcd_a;
  const int a_lo = (int)((int64_t)xa * g.tiles_a / g.xcd_a);
  const int na = (int)((int64_t)(xa + 1) * g.tiles_a / g.xcd_a) - a_lo;
  const int b_lo = (int)((int64_t)xb * g.tiles_b / xb_parts);
  const int nb = (int)((int64_t)(xb + 1) * g.tiles_b / xb_parts) - b_lo;
  if (local >= na * nb) return false;
  // within the XCD: groups of group_b B tiles, each walked with all of the XCD's A tiles
  const int gsz = g.group_b * na;
  const int grp = local / gsz;
  const int r = local - grp * gsz;
  const int gb = min(g.group_b, nb - grp * g.group_b);
  ta = a_lo + r / gb;
  tb = b_lo + grp * g.group_b + r % gb;
  return true;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// A buffer offset beyond every range used here: a buffer load from it returns zeros.
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kMaxRange = 0x7ffffff0u;

// Raw buffer resource over [base, base + bytes): loads at offsets past `bytes` return 0,
// which zero-fills the rows and K columns beyond the operand without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes > (int64_t)kMaxRange ? kMaxRange : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Row-major operand, k contiguous: rows [row0, row0 + 256) of a matrix with `ld` elements
// per row; one K step covers 128 bytes of k.  Thread tid moves chunk tid % 8 of rows
// tid / 8 + 32 p.  Rows past the matrix and chunks at or past `kend` read as zero.
template <typename T>
struct DirectTile {
  uint4 v[8];
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t vrow;      // byte offset of this thread's first row and chunk
  uint32_t rstride;   // bytes between the rows one thread moves (32 rows)
  int kc;             // k of this thread's chunk within a K step
  __device__ __forceinline__ void init(const T* base, int64_t ld, int row0, int nrows, int tid) {
    const int rows = max(0, min(nrows - row0, kTile));
    rsrc = make_rsrc(base + (int64_t)row0 * ld, (int64_t)rows * ld * (int64_t)sizeof(T));
    vrow = (uint32_t)((tid >> 3) * ld * (int64_t)sizeof(T)) + (uint32_t)((tid & 7) * 16);
    rstride = (uint32_t)(32 * ld * (int64_t)sizeof(T));
    kc = (tid & 7) * (16 / (int)sizeof(T));
  }
  __device__ __forceinline__ void load(int k0, int kend) {
    const uint32_t soff = (uint32_t)k0 * (uint32_t)sizeof(T);
    const uint32_t base = k0 + kc < kend ? vrow : kOOB;
#pragma unroll
    for (int p = 0; p < 8; ++p) v[p] = bload(rsrc, base == kOOB ? kOOB : base + p * rstride, soff);
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < 8; ++p)
      *reinterpret_cast<uint4*>(lds + lds_off((tid >> 3) + 32 * p, tid & 7)) = v[p];
  }
};

// Transposed operand of the dH GEMM: LDS row d holds W[k0 .. k0 + 128 bytes, d0 + d].
template <typename T>
struct TransTile;

template <>
struct TransTile<__bf16> {
  uint4 v[8];  // 8 vocabulary rows x 8 hidden columns
  const __bf16* W;
  int64_t D;
  int d0;
  uint32_t voff;  // this thread's block: row 8 (tid / 32), column 8 (tid % 32); kOOB past D
  __device__ __forceinline__ void init(const __bf16* W_, int64_t D_, int d0_, int tid) {
    W = W_;
    D = D_;
    d0 = d0_;
    const int col = 8 * (tid & 31);
    voff = d0 + col < D ? (uint32_t)((8 * (tid >> 5)) * D * 2 + col * 2) : kOOB;
  }
  __device__ __forceinline__ void load(int k0, int kend) {
    const int64_t rows = min(kend - k0, 64);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(W + (int64_t)k0 * D + d0, (rows * D - d0) * 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bload(r, voff, (uint32_t)(e * D * 2));  // kOOB + soff stays out of range
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
    const int b = tid & 31, a = tid >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = u4get(v[2 * q], i >> 1), hi = u4get(v[2 * q + 1], i >> 1);
        w[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<uint4*>(lds + lds_off(8 * b + i, a)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
};

template <>
struct TransTile<float> {
  uint4 v[8];  // 4 vocabulary rows x 8 hidden columns (two chunks per row)
  const float* W;
  int64_t D;
  int d0;
  uint32_t voff0, voff1;  // first and second chunk of this thread's block; kOOB past D
  __device__ __forceinline__ void init(const float* W_, int64_t D_, int d0_, int tid) {
    W = W_;
    D = D_;
    d0 = d0_;
    const int col = 8 * (tid & 31);
    const uint32_t row = (uint32_t)((4 * (tid >> 5)) * D * 4);
    voff0 = d0 + col < D ? row + col * 4 : kOOB;
    voff1 = d0 + col + 4 < D ? row + col * 4 + 16 : kOOB;
  }
  __device__ __forceinline__ void load(int k0, int kend) {
    const int64_t rows = min(kend - k0, 32);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(W + (int64_t)k0 * D + d0, (rows * D - d0) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bload(r, voff0, (uint32_t)(e * D * 4));  // kOOB + soff stays out of range
      v[2 * e + 1] = bload(r, voff1, (uint32_t)(e * D * 4));
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
    const int b = tid & 31, a = tid >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int h = i >> 2, c = i & 3;
      *reinterpret_cast<uint4*>(lds + lds_off(8 * b + i, a)) =
          make_uint4(u4get(v[h], c), u4get(v[2 + h], c), u4get(v[4 + h], c), u4get(v[6 + h], c));
    }
  }
};

// ---- bf16 GEMMs: 256 x 256 workgroup tiles, four waves side by side (wave w owns
// B rows 64 w .. 64 w + 63 and all 256 A rows).  Only the A tile goes through LDS,
// a 4-stage ring of 32 bf16 of K per stage (16 KB); each wave streams its own B rows
// from global memory straight into registers, from a fragment-major copy of B in which
// every 32-row x 16-k MFMA operand fragment is one contiguous 1 KB block.  The A tile
// enters the ring by direct-to-LDS loads from the same layout when the workspace holds a
// fragment-major copy of W, W^T or the dW operands (DmaFragA), else from row-major W
// (DmaTileA) or transposed in registers on the way (TransTileA).  Per 32 of K a workgroup
// moves 32 KB from L2 (16 KB of A, 4 x 4 KB of B) for 4.2 MFLOP.
constexpr int kTA = kTileA16;           // A rows per workgroup
constexpr int kTB = kTileB16;           // B rows per workgroup
constexpr int kFB = kTB / 32;           // B fragments (32 rows) per tile
constexpr int kFA = kTA / 32;           // A fragments per tile
constexpr int kFBW = kFB / 4;           // B fragments per wave
constexpr int kBK16 = 32;               // K per ring stage
constexpr int kStagesA = 4;
constexpr int kAStageBytes = kTA * kBK16 * 2;  // 16 KB
constexpr int kDmaA = kAStageBytes / 1024 / 4; // 1 KB direct-to-LDS loads per wave per stage
static_assert(kTA == 256 && kTB == 256, "the wave layout below assumes 256 x 256 tiles");

// Ring stage layout: two logical rows share one 128-byte LDS row (row R in LDS row
// R / 2, chunk 4 (R % 2) + c for its 16-byte k chunk c); the chunk index is XORed with
// f2(R / 2), so that the 32 consecutive rows of an MFMA fragment read, and each 1 KB
// direct-to-LDS write, touch distinct banks for 32- and 64-bank LDS.
__device__ __forceinline__ int f2(int y) { return (y & 3) ^ ((y >> 1) & 3); }
__device__ __forceinline__ int lds_off2(int R, int c) {
  const int y = R >> 1;
  return y * 128 + (((4 * (R & 1) + c) ^ f2(y)) << 4);
}
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Byte offset of element (row, k) in the fragment-major layout of a B operand with
// ks_count = ceil(K / 16) k steps: [row / 256][k / 16][(row % 256) / 32][lane][8 elements]
// with lane = row % 32 + 32 ((k % 16) / 8).
__device__ __forceinline__ int64_t frag_off(int row, int k, int ks_count) {
  const unsigned r = (unsigned)row;
  return ((((int64_t)(r / kTB) * ks_count + (k >> 4)) * kFB + ((r % kTB) >> 5)) * 64 +
          ((r & 31) + 32 * ((k >> 3) & 1))) * 16 + (k & 7) * 2;
}

// Row-major bf16 A operand (k contiguous) moved straight into the ring: wave w issues
// kDmaA buffer loads per stage, load j filling 1 KB (16 logical rows 64 w + 16 j ..);
// lane i of a load fills 16 bytes at i * 16, so it fetches the row and chunk the
// swizzle places there (the swizzle depends on the LDS row modulo 8 only).
struct DmaTileA {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lane_off;  // byte offset of this lane's row and chunk from the tile base
  uint32_t jstride;   // bytes between the 16-row groups of the wave's loads
  int kc;             // k of this lane's chunk within a stage
  int w;              // wave index (uniform)
  __device__ __forceinline__ void init(const __bf16* base, int64_t ld, int row0, int nrows, int tid) {
    const int rows = max(0, min(nrows - row0, kTA));
    rsrc = make_rsrc(base + (int64_t)row0 * ld, (int64_t)rows * ld * 2);
    const int i = tid & 63;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int y = i >> 3;
    const int cp = (i & 7) ^ f2(y);
    const int dR = 2 * y + (cp >> 2);
    const int c = cp & 3;
    lane_off = (uint32_t)(((kTA / 4) * w + dR) * ld * 2 + 16 * c);
    jstride = (uint32_t)(16 * ld * 2);
    kc = 8 * c;
  }
  __device__ __forceinline__ void issue(char* lds_stage, int k0, int kend) const {
    const uint32_t v = k0 + kc < kend ? lane_off : kOOB;
#pragma unroll
    for (int j = 0; j < kDmaA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(lds_stage + (kDmaA * w + j) * 1024), 16, v,
                                               (uint32_t)(j * jstride + k0 * 2), 0, 0);
  }
};

// Fragment-major bf16 A operand (the copies of W and W^T) moved straight into the ring:
// with the layout [row / 256][k / 16][(row % 256) / 32][lane][8 elements], one ring stage
// of a 256-row tile (two k steps) is 16 KB of consecutive bytes, so wave w issues kDmaA
// loads of one contiguous kilobyte each (fragments 4 w .. 4 w + 3 of the stage, k step
// first), whole cache lines.  The stage in LDS keeps that order: fragment f of k step kk at
// (8 kk + f) KB, lane l's 16 bytes at 16 l.  The buffer range ends with the tile's last k
// step, so loads past K read zeros; stages at or past `kend` (the split's end, a multiple
// of the stage) read zeros too.
struct DmaFragA {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lane_off;  // 16 l
  int w;              // wave index (uniform)
  int wrap;           // k step at which the operand's k index starts again at 0 (0: never)
  int koff;           // k steps before the copy's first (a band of W^T)
  __device__ __forceinline__ void init(const void* Af, int ks_count, int tile, int tid, int wrap_ks = 0,
                                       int koff_ks = 0) {
    const int64_t bytes = (int64_t)ks_count * kFA * 1024;
    rsrc = make_rsrc(reinterpret_cast<const char*>(Af) + (int64_t)tile * bytes, bytes);
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane_off = (uint32_t)((tid & 63) * 16);
    wrap = wrap_ks;
    koff = koff_ks;
  }
  __device__ __forceinline__ void issue(char* lds_stage, int k0, int kend) const {
    const uint32_t v = k0 < kend ? lane_off : kOOB;
    const int kr = (k0 >> 4) - koff;
    const int ks = (wrap > 0 && kr >= wrap) ? kr - wrap : kr;
    const uint32_t base = (uint32_t)ks * (kFA * 1024);
#pragma unroll
    for (int j = 0; j < kDmaA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(lds_stage + (kDmaA * w + j) * 1024), 16, v,
                                               base + (uint32_t)((kDmaA * w + j) * 1024), 0, 0);
  }
};

// Transposed A operand of the dH GEMM (W read as W^T): lane (h = lane % 2, q = lane / 2)
// of wave c loads vocabulary rows 8c + 4h .. + 3 of the stage at hidden columns
// d0 + 128 p + 4q .. + 3 (p = 0, 1), transposes each 4 x 4 block in registers and
// writes four 8-byte half chunks per block; in store t it writes column 4q + (t + q / 4) % 4,
// which keeps the 64 lanes of a store on distinct banks.
struct TransTileA {
  uint2 v[2][4];
  const __bf16* W;
  int64_t D;
  int d0, c, h, q;
  uint32_t voff[2];
  __device__ __forceinline__ void init(const __bf16* W_, int64_t D_, int d0_, int tid) {
    W = W_;
    D = D_;
    d0 = d0_;
    const int lane = tid & 63;
    c = tid >> 6;
    h = lane & 1;
    q = lane >> 1;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      voff[p] = d0 + 128 * p + 4 * q < D ? (uint32_t)(((8 * c + 4 * h) * D + 128 * p + 4 * q) * 2) : kOOB;
  }
  // k0 in the (possibly doubled) reduction; wrap: where the vocabulary index starts again at 0
  // (0: never); rows at or past V, or at or past kend, read as zero.
  __device__ __forceinline__ void load(int k0, int kend, int wrap, int V) {
    const int kv = (wrap > 0 && k0 >= wrap) ? k0 - wrap : k0;
    const int64_t rows = min(min(kend - k0, kBK16), V - kv);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(W + (int64_t)kv * D + d0, rows > 0 ? (rows * D - d0) * 2 : 0);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the scalar offset must stay uniform; kOOB + e * D * 2 is still past the range
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff[p], (uint32_t)(e * D * 2), 0);
        v[p][e] = make_uint2(x.x, x.y);
      }
  }
  __device__ __forceinline__ void store(char* lds_stage) const {
    const int r = (q >> 2) & 3;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint2 o[4];  // o[i]: vocabulary rows 4h .. 4h + 3 of hidden column 128 p + 4q + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a0 = (i < 2) ? v[p][0].x : v[p][0].y, a1 = (i < 2) ? v[p][1].x : v[p][1].y;
        const uint32_t a2 = (i < 2) ? v[p][2].x : v[p][2].y, a3 = (i < 2) ? v[p][3].x : v[p][3].y;
        o[i] = make_uint2(halves(a0, a1, i & 1), halves(a2, a3, i & 1));
      }
      if (r & 1) {
        const uint2 t0 = o[0];
        o[0] = o[1]; o[1] = o[2]; o[2] = o[3]; o[3] = t0;
      }
      if (r & 2) {
        uint2 t0 = o[0]; o[0] = o[2]; o[2] = t0;
        t0 = o[1]; o[1] = o[3]; o[3] = t0;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<uint2*>(lds_stage + lds_off2(128 * p + 4 * q + ((t + r) & 3), c) + 8 * h) = o[t];
    }
  }
};

// A fragments of one 16-wide k step (kk = 0, 1) of a ring stage: rows 32 f + l % 32,
// k = 16 kk + 8 (l / 32) + 0..7.
__device__ __forceinline__ void a_frags(const char* As, int kk, int lane, bf16x8 (&a)[kFA]) {
  const int c = 2 * kk + (lane >> 5);
#pragma unroll
  for (int f = 0; f < kFA; ++f)
    a[f] = *reinterpret_cast<const bf16x8*>(As + lds_off2(f * 32 + (lane & 31), c));
}

// The same from a stage filled by DmaFragA: one contiguous kilobyte per fragment.
__device__ __forceinline__ void a_frags_f(const char* As, int kk, int lane, bf16x8 (&a)[kFA]) {
#pragma unroll
  for (int f = 0; f < kFA; ++f)
    a[f] = *reinterpret_cast<const bf16x8*>(As + (kk * kFA + f) * 1024 + lane * 16);
}

// This wave's B fragments of one stage (2 k steps x 2 fragments) from the fragment-major
// copy.  K steps past the end are clamped to the last one: the copy holds finite values
// everywhere and the A operand of those stages is zero, so they add nothing.
__device__ __forceinline__ void b_load(const char* Bw, int ks, int ks_count, bf16x8 (&b)[2][kFBW]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const char* p = Bw + (int64_t)min(ks + kk, ks_count - 1) * (kFB * 1024);
#pragma unroll
    for (int f = 0; f < kFBW; ++f) b[kk][f] = *reinterpret_cast<const bf16x8*>(p + f * 1024);
  }
}

__device__ __forceinline__ void mma16(const bf16x8 (&a)[kFA], const bf16x8 (&b)[kFBW],
                                      floatx16 (&acc)[kFA][kFBW]) {
#pragma unroll
  for (int j = 0; j < kFBW; ++j)
#pragma unroll
    for (int i = 0; i < kFA; ++i)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmLgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }
constexpr int kWaitAll = 0x0070;

// One LDS stage (128 bytes of K per row) of MFMA work for a wave's 128 x 128 sub-tile.
// Lane l supplies row (l % 32) of each 32-row block and k = 8 (l / 32) + 0..7 of each
// 16-wide k step, for both operands alike.  The fragments of k step i + 1 are read from
// LDS while the 16 MFMAs of step i run.
template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  __device__ __forceinline__ static void frags(const char* As, const char* Bs, int kk, int wm, int wn, int lane,
                                               bf16x8 (&a)[4], bf16x8 (&b)[4]) {
    const int c = 2 * kk + (lane >> 5);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      a[f] = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * 128 + f * 32 + (lane & 31), c));
      b[f] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wn * 128 + f * 32 + (lane & 31), c));
    }
  }
  __device__ __forceinline__ static void mma(const bf16x8 (&a)[4], const bf16x8 (&b)[4], floatx16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  __device__ __forceinline__ static void stage(const char* As, const char* Bs, floatx16 (&acc)[4][4],
                                               int wm, int wn, int lane) {
    bf16x8 a[2][4], b[2][4];
    frags(As, Bs, 0, wm, wn, lane, a[0], b[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) frags(As, Bs, kk + 1, wm, wn, lane, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][i], b[kk & 1][j], acc[i][j], 0, 0, 0);
    }
  }
};

template <>
struct Mma<float> {
  __device__ __forceinline__ static void stage(const char* As, const char* Bs, floatx16 (&acc)[4][4],
                                               int wm, int wn, int lane) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = 4 * kk + 2 * (lane >> 5);
      float4 a[4][2], b[4][2];
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          a[f][h] = *reinterpret_cast<const float4*>(As + lds_off(wm * 128 + f * 32 + (lane & 31), c + h));
          b[f][h] = *reinterpret_cast<const float4*>(Bs + lds_off(wn * 128 + f * 32 + (lane & 31), c + h));
        }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float av = e < 4 ? a[i][0][e] : a[i][1][e - 4];
            const float bv = e < 4 ? b[j][0][e] : b[j][1][e - 4];
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[i][j], 0, 0, 0);
          }
    }
  }
};

// Store 4 consecutive elements (fp32 values) to a row of T.
__device__ __forceinline__ void store4(__bf16* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(a, b), pack_bf16(c, d));
}
__device__ __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void load4(const __bf16* src, float (&o)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(src);
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
}
__device__ __forceinline__ void load4(const float* src, float (&o)[4]) {
  const float4 u = *reinterpret_cast<const float4*>(src);
  o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
}

// fp32 GEMMs (inputs kept in fp32): 256 x 256 tiles, 2 x 2 waves of 128 x 128, K staged
// through a double-buffered LDS tile of 128-byte rows.  Accumulator element (i, j, r) of
// lane l: A-row wm*128 + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4, B-row (token) wn*128 + 32 j + l % 32.
template <typename T, int KIND>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kTileBytes];
  int ta, tb;
  if (!map_tile(g, ta, tb)) return;
  constexpr int BK = 128 / (int)sizeof(T);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int ks = 0, tile_a = ta;
  if (KIND == KIND_DH) {
    ks = ta / g.tiles_a_base;
    tile_a = ta - ks * g.tiles_a_base;
  }
  const int row_a0 = tile_a * kTile;
  const int row_b0 = tb * kTile;
  const int k_begin = ks * g.k_len;
  const int k_end = min(g.K, k_begin + g.k_len);
  const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const T* A = reinterpret_cast<const T*>(g.a);
  const T* B = reinterpret_cast<const T*>(g.b);
  // stage s: A operand at smem + s * 64 KB, B operand 32 KB after it

  {
    using ALoader = typename std::conditional<KIND == KIND_DH, TransTile<T>, DirectTile<T>>::type;
    ALoader la;
    DirectTile<T> lb;
    if constexpr (KIND == KIND_DH) la.init(A, g.lda, row_a0, tid);
    else la.init(A, g.lda, row_a0, g.a_rows, tid);
    lb.init(B, g.ldb, row_b0, g.b_rows, tid);
    if (nk > 0) {
      la.load(k_begin, k_end);
      lb.load(k_begin, k_end);
      la.store(smem, tid);
      lb.store(smem + kTileBytes, tid);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
          const int k0 = k_begin + (kt + 1) * BK;
          la.load(k0, k_end);
          lb.load(k0, k_end);
        }
        char* sc = smem + cur * (2 * kTileBytes);
        char* sn = smem + (cur ^ 1) * (2 * kTileBytes);
        Mma<T>::stage(sc, sc + kTileBytes, acc, wm, wn, lane);
        if (more) {
          la.store(sn, tid);
          lb.store(sn + kTileBytes, tid);
        }
        __syncthreads();
      }
    }
  }

  const int hi = lane >> 5;     // which 4-row half of each 8-row group this lane holds
  const int col = lane & 31;

  if constexpr (KIND == KIND_LSE || KIND == KIND_PROBS) {
    if (g.lm.cap_in > 0.0f) {  // softcap: the accumulators become v = tanh(cap_in x)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = tanh_fast(acc[i][j][r] * g.lm.cap_in);
    }
  }
  if constexpr (KIND == KIND_LSE) {
    // Per token: max and sum of exp over this tile's vocabulary rows (those < V).
    float* red_m = reinterpret_cast<float*>(smem);
    float* red_s = red_m + 2 * kTile;
    const bool full = row_a0 + kTile <= g.a_rows;
    const int vbase = row_a0 + wm * 128 + 4 * hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = vbase + 32 * i + 8 * (r >> 2) + (r & 3);
          if (full || v < g.a_rows) mx = fmaxf(mx, acc[i][j][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float zmax = mx * g.lm.zscale;  // zscale > 0, so this is the max of z
      float s = 0.0f;
      if (mx > -INFINITY) {
        const float c1 = g.lm.zscale * kLog2e, c0 = -zmax * kLog2e;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int v = vbase + 32 * i + 8 * (r >> 2) + (r & 3);
            if (full || v < g.a_rows) s += __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], c1, c0));
          }
      }
      s += __shfl_xor(s, 32);
      if (hi == 0) {
        red_m[wm * kTile + wn * 128 + 32 * j + col] = zmax;
        red_s[wm * kTile + wn * 128 + 32 * j + col] = s;
      }
    }
    __syncthreads();
    const int tok = row_b0 + tid;
    if (tok < g.b_rows) {
      const float m0 = red_m[tid], m1 = red_m[kTile + tid];
      const float M = fmaxf(m0, m1);
      float S = 0.0f;
      if (m0 > -INFINITY) S += red_s[tid] * __builtin_amdgcn_exp2f((m0 - M) * kLog2e);
      if (m1 > -INFINITY) S += red_s[kTile + tid] * __builtin_amdgcn_exp2f((m1 - M) * kLog2e);
      g.pm[(int64_t)tok * g.tiles_a + tile_a] = M;
      g.ps[(int64_t)tok * g.tiles_a + tile_a] = S;
    }
  } else if constexpr (KIND == KIND_PROBS) {
    // P'[token, v] = exp(z - lse[token]) (times 1 - v^2 with a softcap) for v < V, written
    // as 4-element vectors (target entries then rewritten by onehot_fix_kernel).
    T* P = reinterpret_cast<T*>(g.p);
    const float c1 = g.lm.zscale * kLog2e;
    const bool cap = g.lm.cap_in > 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = row_b0 + wn * 128 + 32 * j + col;
      if (tok >= g.b_rows) continue;
      const float c0 = -g.lse[tok] * kLog2e;
      T* prow = P + (int64_t)tok * g.ldp;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v0 = row_a0 + wm * 128 + 32 * i + 8 * q + 4 * hi;
          float e[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x = acc[i][j][4 * q + u];
            e[u] = __builtin_amdgcn_exp2f(fmaf(x, c1, c0));
            if (cap) e[u] *= 1.0f - x * x;
          }
          if (v0 + 4 <= g.V) {
            store4(prow + v0, e[0], e[1], e[2], e[3]);
          } else if (v0 < g.ldp) {
            // the row's padding up to the 16-byte boundary is written as zeros: the dH
            // GEMM reads whole 16-byte chunks
            store4(prow + v0, v0 < g.V ? e[0] : 0.0f, v0 + 1 < g.V ? e[1] : 0.0f, v0 + 2 < g.V ? e[2] : 0.0f,
                   v0 + 3 < g.V ? e[3] : 0.0f);
          }
        }
    }
  } else {
    // dH[token, d] = (g / tau) (W[y, d] - acc), or the raw fp32 partial when split.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = row_b0 + wn * 128 + 32 * j + col;
      if (tok >= g.b_rows) continue;
      if (g.ksplit > 1) {
        float* dst = g.part + ((int64_t)ks * g.b_rows + tok) * g.D;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d0 = row_a0 + wm * 128 + 32 * i + 8 * q + 4 * hi;
            if (d0 < g.D)
              *reinterpret_cast<float4*>(dst + d0) =
                  make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
        continue;
      }
      const TokGrad tg = tok_grad(g.g, g.targets, g.zy, g.V, g.lm, tok, true);
      const bool live = tg.live;
      T* dst = reinterpret_cast<T*>(g.dh) + (int64_t)tok * g.D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d0 = row_a0 + wm * 128 + 32 * i + 8 * q + 4 * hi;
          if (d0 >= g.D) continue;
          float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (live) {
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = -tg.c * acc[i][j][4 * q + u];
          }
          store4(dst + d0, o[0], o[1], o[2], o[3]);
        }
    }
  }
}

// bf16 GEMMs on 256 x 256 tiles.  Accumulator element (i, j, r) of lane l of wave w:
// A-row 32 i + 8 (r / 4) + 4 (l / 32) + r % 4 of the tile, B-row (token) 64 w + 32 j + l % 32.
// Iteration kt computes ring stage kt in two 16-wide k steps: the loads of A stage kt + 3
// and of this wave's B stage kt + 3 and the A fragments of step 1 are issued under the
// MFMAs of step 0; then the A loads of stage kt + 1 are waited for, a barrier publishes
// every wave's, and the A fragments of stage kt + 1, step 0 are read under the MFMAs of
// step 1.  A ring slot is refilled only after the barrier that follows its last read.
//
// Epilogue of a bf16 GEMM tile: straight-line code over the accumulators.  Rows of the last
// vocabulary tile at or past V entered the main loop at -inf and stayed there (those rows of
// W read as zero), so the logits epilogues need no masks: they add nothing to the max, their
// exp is 0, and with a softcap they stay -inf.  Groups of 8 rows (32 i + 8 q + 0..7 of the
// tile) past the stored width are skipped by uniform scalar tests.
template <int KIND, bool kSplit, bool kCap, bool kOut32, bool kAcc>
__device__ __forceinline__ void gemm16_epi(const GemmArgs& g, floatx16 (&acc)[kFA][kFBW], int ks, int tile_a,
                                           int tb) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_a0 = tile_a * kTA;
  const int row_b0 = tb * kTB;
  const int hi = lane >> 5;
  const int col = lane & 31;
  constexpr bool kLogits = KIND == KIND_LSE || KIND == KIND_PROBS || KIND == KIND_LSES;
  // With a softcap the accumulators of token block j become v = tanh(cap_in x) (-inf stays
  // -inf) at the start of that block's epilogue, one block at a time.
  auto cap_block = [&](int j) {
    if constexpr (kLogits && kCap) {
#pragma unroll
      for (int i = 0; i < kFA; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = acc[i][j][r];
          const float t = tanh_fast(x * g.lm.cap_in);
          acc[i][j][r] = x == -INFINITY ? x : t;
        }
        __builtin_amdgcn_sched_barrier(0);  // 16 values in flight at a time
      }
    }
  };
  if constexpr (KIND == KIND_LSE || KIND == KIND_LSES) {
    // Per token: max and sum of exp over this tile's vocabulary rows below V; KIND_LSES also
    // keeps d = z - max (fp16, rounded to nearest) in the fragment-major layout of the
    // probabilities (-inf past V).
#pragma unroll
    for (int j = 0; j < kFBW; ++j) {
      cap_block(j);
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < kFA; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));  // finite: row 0 of the tile is below V
      const float zmax = mx * g.lm.zscale;  // zscale > 0, so this is the max of z
      const int tok = row_b0 + 64 * w + 32 * j + col;
      if (g.zy_out) {
        // The target logit z[t, y_t] from the same accumulator the max and the sum use: the lane
        // holding tile row y_t - row_a0 (rows 32 i + 8 q + 4 hi + u) picks it out.  A tile holds a
        // given token's target with probability 256 / V, so this branch is rare and divergent.
        const int tloc = tok < g.b_rows ? g.targets[tok] - row_a0 : -1;
        if (tloc >= 0 && tloc < kTA && ((tloc >> 2) & 1) == hi) {
          float z = 0.0f;
#pragma unroll
          for (int i = 0; i < kFA; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) z = 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3) == tloc ? acc[i][j][r] : z;
          g.zy_out[tok] = z * g.lm.zscale;
        }
      }
      if constexpr (KIND == KIND_LSES) {
        char* P = reinterpret_cast<char*>(g.p);
        const int vpad = g.v_ks * 16 - row_a0;  // uniform; multiple of 16
#pragma unroll
        for (int i = 0; i < kFA; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int g0 = 32 * i + 8 * q;
            if (__builtin_expect(g0 >= vpad, 0)) continue;
            float d[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) d[u] = fmaf(acc[i][j][4 * q + u], g.lm.zscale, -zmax);
            *reinterpret_cast<uint2*>(P + frag_off(tok, row_a0 + g0 + 4 * hi, g.p_ks)) =
                make_uint2(pack_f16(d[0], d[1]), pack_f16(d[2], d[3]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const float c1 = g.lm.zscale * kLog2e, c0 = -zmax * kLog2e;
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < kFA; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], c1, c0));
      sum += __shfl_xor(sum, 32);
      if (hi == 0 && tok < g.b_rows) {
        g.pm[(int64_t)tok * g.tiles_a + tile_a] = zmax;
        g.ps[(int64_t)tok * g.tiles_a + tile_a] = sum;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (KIND == KIND_PROBS) {
    // P'[token, v] = exp(z - lse[token]) (times 1 - v^2 with a softcap) into the
    // fragment-major copy used as the B operand of the dH GEMM (the target entries are
    // then rewritten by onehot_fix_kernel); the vocabulary padding up to the next 16 is
    // written as zeros.  Rows of the copy past the chunk's tokens are written too (every
    // consumer ignores them).
    char* P = reinterpret_cast<char*>(g.p);
    const int vpad = g.v_ks * 16 - row_a0;  // uniform; multiple of 16
    const float c1 = g.lm.zscale * kLog2e;
#pragma unroll
    for (int j = 0; j < kFBW; ++j) {
      cap_block(j);
      const int tok = row_b0 + 64 * w + 32 * j + col;
      const float c0 = -(tok < g.b_rows ? g.lse[tok] : 0.0f) * kLog2e;
#pragma unroll
      for (int i = 0; i < kFA; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g0 = 32 * i + 8 * q;
          if (__builtin_expect(g0 >= vpad, 0)) continue;
          float e[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x = acc[i][j][4 * q + u];
            e[u] = __builtin_amdgcn_exp2f(fmaf(x, c1, c0));
            if constexpr (kCap) e[u] = e[u] != 0.0f ? e[u] * (1.0f - x * x) : 0.0f;  // past V: x = -inf
          }
          const uint32_t h01 = pack_bf16(e[0], e[1]), h23 = pack_bf16(e[2], e[3]);
          *reinterpret_cast<uint2*>(P + frag_off(tok, row_a0 + g0 + 4 * hi, g.p_ks)) = make_uint2(h01, h23);
          if constexpr (kOut32) {  // lo = e - hi, the part the bf16 rounding dropped
            *reinterpret_cast<uint2*>(P + frag_off(tok, g.lo_ks * 16 + row_a0 + g0 + 4 * hi, g.p_ks)) =
                make_uint2(pack_bf16(e[0] - bf16_lo(h01), e[1] - bf16_hi(h01)),
                           pack_bf16(e[2] - bf16_lo(h23), e[3] - bf16_hi(h23)));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if constexpr (KIND == KIND_DW) {
    // dW[v, d] = acc (first chunk) or dW[v, d] + acc, fp32, with the hidden units d as the A
    // rows and the band's vocabulary entries v as the B rows: acc = sum_t (-c_t H[t, d]) Q[t, v].
    // A lane's 4 consecutive accumulator rows are 4 consecutive floats of a dW row.
    float* dw = g.dw;
    const int drem = g.D - row_a0;  // uniform; multiple of 8
#pragma unroll
    for (int j = 0; j < kFBW; ++j) {
      const int v = row_b0 + 64 * w + 32 * j + col;
      if (v >= g.V) continue;
      float* row = dw + (int64_t)v * g.D;
#pragma unroll
      for (int i = 0; i < kFA; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (__builtin_expect(32 * i + 8 * q >= drem, 0)) continue;
          float4* p = reinterpret_cast<float4*>(row + row_a0 + 32 * i + 8 * q + 4 * hi);
          float4 o = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          if (g.accumulate) {
            const float4 x = *p;
            o.x += x.x;
            o.y += x.y;
            o.z += x.z;
            o.w += x.w;
          }
          *p = o;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // dH[token, d] = -c acc with acc = sum_v Q[token, v] W[v, d] (+0 rows for tokens without
    // a gradient), or the raw fp32 partial when split.
    const int drem = g.D - row_a0;  // uniform; multiple of 8
#pragma unroll
    for (int j = 0; j < kFBW; ++j) {
      const int tok = row_b0 + 64 * w + 32 * j + col;
      const bool ok = tok < g.b_rows;
      if constexpr (kSplit) {
        float* dst = g.part + ((int64_t)ks * g.b_rows + (ok ? tok : 0)) * g.D;
#pragma unroll
        for (int i = 0; i < kFA; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (__builtin_expect(32 * i + 8 * q >= drem, 0)) continue;
            const int d0 = row_a0 + 32 * i + 8 * q + 4 * hi;
            float4 o =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            if (ok) {
              float4* pp = reinterpret_cast<float4*>(dst + d0);
              if constexpr (kAcc) {  // a later band of a banded W^T
                const float4 x = *pp;
                o.x = x.x + o.x;
                o.y = x.y + o.y;
                o.z = x.z + o.z;
                o.w = x.w + o.w;
              }
              *pp = o;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      const TokGrad tg = tok_grad(g.g, g.targets, g.zy, g.V, g.lm, tok, ok);
      const float nc = -tg.c;
      if constexpr (kOut32) {  // fp32 dH (the probabilities were read as hi + lo pairs)
        float* dst = reinterpret_cast<float*>(g.dh) + (int64_t)(ok ? tok : 0) * g.D;
#pragma unroll
        for (int i = 0; i < kFA; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (__builtin_expect(32 * i + 8 * q >= drem, 0)) continue;
            const int d0 = row_a0 + 32 * i + 8 * q + 4 * hi;
            float o[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = tg.live ? nc * acc[i][j][4 * q + u] : 0.0f;
            if (ok) store4(dst + d0, o[0], o[1], o[2], o[3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        __bf16* dst = reinterpret_cast<__bf16*>(g.dh) + (int64_t)(ok ? tok : 0) * g.D;
#pragma unroll
        for (int i = 0; i < kFA; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (__builtin_expect(32 * i + 8 * q >= drem, 0)) continue;
            const int d0 = row_a0 + 32 * i + 8 * q + 4 * hi;
            float o[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = tg.live ? nc * acc[i][j][4 * q + u] : 0.0f;
            if (ok) store4(dst + d0, o[0], o[1], o[2], o[3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

// One kernel holds one tile body: the softcap (kCap), the A operand's layout (kFragA), a
// split vocabulary (kSplit, dH: fp32 partials), fp32 dH (kOut32) and partials added to
// instead of written (kAcc: the later bands of a banded W^T) are chosen on the host, so
// register allocation covers a single main loop and epilogue.
template <int KIND, bool kSplit, bool kCap, bool kFragA, bool kOut32, bool kAcc>
__device__ __forceinline__ void gemm16_tile(const GemmArgs& g, char* smem, int ks, int tile_a, int tb) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool kTrans = KIND == KIND_DH;  // A transposed in registers
  const int row_a0 = tile_a * kTA;
  const int row_b0 = tb * kTB;
  const int k_begin = g.k_base + ks * g.k_len;
  const int k_end = min(g.K, k_begin + g.k_len);
  const int nk = k_end > k_begin ? (k_end - k_begin + kBK16 - 1) / kBK16 : 0;

  floatx16 acc[kFA][kFBW];
#pragma unroll
  for (int i = 0; i < kFA; ++i)
#pragma unroll
    for (int j = 0; j < kFBW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if constexpr (KIND == KIND_LSE || KIND == KIND_PROBS || KIND == KIND_LSES) {
    if (row_a0 + kTA > g.V) {  // uniform: the last vocabulary tile; its rows past V start at -inf
      const int vlim_l = g.V - row_a0 - 4 * (lane >> 5);  // A-row 32 i + 8 (r / 4) + 4 (l / 32) + r % 4
#pragma unroll
      for (int i = 0; i < kFA; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v0 = 32 * i + 8 * (r >> 2) + (r & 3) < vlim_l ? 0.0f : -INFINITY;
#pragma unroll
          for (int j = 0; j < kFBW; ++j) acc[i][j][r] = v0;
        }
    }
  }

  const __bf16* A = reinterpret_cast<const __bf16*>(g.a);
  // this wave's 64 rows of the B tile in the fragment-major copy
  const char* Bw =
      reinterpret_cast<const char*>(g.b) + (int64_t)tb * g.b_ks * kFB * 1024 + kFBW * w * 1024 + lane * 16;
  const int ks0 = k_begin >> 4;
  using ATile = typename std::conditional<kTrans, TransTileA,
                                          typename std::conditional<kFragA, DmaFragA, DmaTileA>::type>::type;
  ATile at;
  if constexpr (kTrans) at.init(A, g.lda, row_a0, tid);
  else if constexpr (kFragA) at.init(g.a, g.a_ks > 0 ? g.a_ks : g.b_ks, tile_a, tid, g.a_wrap, g.a_koff);
  else at.init(A, g.lda, row_a0, g.a_rows, tid);
  auto afr = [&](const char* As, int kk, bf16x8 (&a)[kFA]) {
    if constexpr (kFragA) a_frags_f(As, kk, lane, a);
    else a_frags(As, kk, lane, a);
  };

  if (nk > 0) {
#pragma unroll
    for (int st = 0; st < kStagesA - 1; ++st) {
      const int k0 = k_begin + st * kBK16;
      if constexpr (kTrans) {
        at.load(k0, k_end, g.a_wrap * 16, g.V);
        at.store(smem + st * kAStageBytes);
      } else {
        at.issue(smem + st * kAStageBytes, k0, k_end);
      }
    }
    bf16x8 bb0[2][kFBW], bb1[2][kFBW], bb2[2][kFBW], bb3[2][kFBW];
    b_load(Bw, ks0, g.b_ks, bb0);
    b_load(Bw, ks0 + 2, g.b_ks, bb1);
    b_load(Bw, ks0 + 4, g.b_ks, bb2);
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
    bf16x8 a0[kFA], a1[kFA];
    afr(smem, 0, a0);
    int slot = 0;
    // loads issued per iteration after A stage kt + 1 (two iterations ago) that may still
    // be in flight when it is waited for: its iteration's B loads and two full iterations
    constexpr int kVmAfterA = 2 * kFBW + 2 * (kDmaA + 2 * kFBW);
    auto step = [&](int kt, bf16x8 (&cur)[2][kFBW], bf16x8 (&nxt)[2][kFBW]) {
      const int slot_n = slot + 1 == kStagesA ? 0 : slot + 1;
      const int slot_f = slot == 0 ? kStagesA - 1 : slot - 1;  // stage kt + kStagesA - 1
      char* sc = smem + slot * kAStageBytes;
      char* sn = smem + slot_n * kAStageBytes;
      char* sf = smem + slot_f * kAStageBytes;
      slot = slot_n;
      const int kf = k_begin + (kt + kStagesA - 1) * kBK16;
      if constexpr (kTrans) at.load(kf, k_end, g.a_wrap * 16, g.V);
      else at.issue(sf, kf, k_end);
      b_load(Bw, ks0 + 2 * (kt + 3), g.b_ks, nxt);
      afr(sc, 1, a1);
      mma16(a0, cur[0], acc);
      // instruction classes: 0x8 MFMA, 0x20 VMEM read, 0x100 DS read, 0x200 DS write
      if constexpr (kTrans) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      } else {
        // the stage's 8 loads and 8 fragment reads spread over all 16 MFMAs
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0(kTrans ? 28 : kVmAfterA));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      afr(sn, 0, a0);
      mma16(a1, cur[1], acc);
      if constexpr (kTrans) at.store(sf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (kTrans) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // four B register buffers rotate, so the loop runs in groups of four stages.  The logits
    // GEMMs (K = D: tens of stages per tile) then run the remaining one to three as single
    // steps; the dH and dW GEMMs (thousands of stages per tile, where the extra code costs
    // registers) run a last padded group whose stages past the end of K read zeros.
    constexpr bool kExactTail = KIND == KIND_LSE || KIND == KIND_PROBS || KIND == KIND_LSES;
    int kt = 0;
    for (; kExactTail ? kt + 4 <= nk : kt < nk; kt += 4) {
      step(kt, bb0, bb3);
      step(kt + 1, bb1, bb0);
      step(kt + 2, bb2, bb1);
      step(kt + 3, bb3, bb2);
    }
    if constexpr (kExactTail) {
      if (kt < nk) {
        step(kt, bb0, bb3);
        if (kt + 1 < nk) {
          step(kt + 1, bb1, bb0);
          if (kt + 2 < nk) step(kt + 2, bb2, bb1);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
  }

  gemm16_epi<KIND, kSplit, kCap, kOut32, kAcc>(g, acc, ks, tile_a, tb);
}

template <int KIND, bool kSplit, bool kCap, bool kFragA, bool kOut32 = false, bool kAcc = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm16_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) char smem[kStagesA * kAStageBytes];
  int ta, tb;
  if (!map_tile(g, ta, tb)) return;
  int ks = 0, tile_a = ta;
  if constexpr (KIND == KIND_DH || KIND == KIND_DHT) {
    ks = ta / g.tiles_a_base;
    tile_a = ta - ks * g.tiles_a_base;
  }
  gemm16_tile<KIND, kSplit, kCap, kFragA, kOut32, kAcc>(g, smem, ks, tile_a, tb);
}

// Fragment-major copy of `rows` rows of a row-major bf16 matrix [rows, K] (ld = K), rows
// past `rows` and k past K zero.  A block moves 32 rows (one fragment row group) x 8 k steps
// (128 elements) through LDS: reads of 128 contiguous bytes per 8 lanes, then per k step
// one contiguous kilobyte of the copy per wave.  The LDS tile keeps row r's 16-byte chunk c
// at chunk c ^ (r % 16), so the column-wise reads of the write phase spread over the banks.
__global__ __launch_bounds__(256) void frag_copy_kernel(const __bf16* __restrict__ X, int rows, int K, int ks_count,
                                                        char* __restrict__ out) {
  __shared__ uint4 tile[32 * 16];
  const int tid = threadIdx.x;
  const int rg = blockIdx.x;               // 32-row group: tile rg / 8, fragment rg % 8
  const int ks0 = blockIdx.y * 8;          // first k step of the block
  {
    const int r = tid >> 3, seg = tid & 7;
    const int row = rg * 32 + r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = seg + 8 * h;
      const int k = ks0 * 16 + 8 * c;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < rows && k < K) v = *reinterpret_cast<const uint4*>(X + (int64_t)row * K + k);
      tile[r * 16 + (c ^ (r & 15))] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = tid + 256 * h;           // unit of the block: k step u / 64, lane u % 64
    const int ks = ks0 + (u >> 6);
    if (ks >= ks_count) continue;
    const int lane = u & 63, r = lane & 31, c = 2 * (u >> 6) + (lane >> 5);
    const int64_t frag = ((int64_t)(rg >> 3) * ks_count + ks) * kFB + (rg & 7);
    *reinterpret_cast<uint4*>(out + frag * 1024 + lane * 16) = tile[r * 16 + (c ^ (r & 15))];
  }
}

// W [V, D] (rows V of a band) into the fragment-major W^T (rows = hidden units, k = vocabulary,
// ks_v k steps).  A block takes 256 vocabulary rows x 64 hidden units: each thread reads 8 rows
// x 8 units (16-byte row pieces, 128 contiguous bytes per 8 lanes), transposes that 8 x 8 block
// with byte permutes into 8 output units (8 vocabulary entries of one hidden unit), and puts
// them at their place in the block's 32 KB of output, staged in LDS; the block then writes
// 16 runs of 2 KB (one k step x the two 32-unit row groups), one contiguous kilobyte per wave
// instruction.  LDS slot s holds unit s ^ ((s >> 4) & 15) of the image, which spreads both the
// scattered unit writes and the consecutive reads over the banks.  Vocabulary rows past V and
// hidden units past D are zeros; k steps at or past ks_v are not written.
__global__ __launch_bounds__(256) void transpose_w_kernel(const __bf16* __restrict__ W, int V, int D, int ks_v,
                                                          char* __restrict__ WTf) {
  __shared__ uint4 img[2048];  // [k step 16][row group 2][unit 64]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int vl = (tid >> 6) * 64 + 8 * (lane >> 3);  // block-relative vocabulary row
  const int dl = 8 * (lane & 7);                       // block-relative hidden unit
  const int v0 = blockIdx.x * 256 + vl;
  const int d0 = blockIdx.y * 64 + dl;
  const bool live = v0 < 16 * ks_v;
  uint4 r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r[i] = live && v0 + i < V && d0 < D ? *reinterpret_cast<const uint4*>(W + (int64_t)(v0 + i) * D + d0)
                                        : make_uint4(0, 0, 0, 0);
  auto slot = [](int u) { return u ^ ((u >> 4) & 15); };
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = u4get(r[2 * m], j >> 1), b = u4get(r[2 * m + 1], j >> 1);
      o[m] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    const int d = dl + j;
    const int u = ((vl >> 4) * 2 + (d >> 5)) * 64 + (d & 31) + 32 * ((vl >> 3) & 1);
    img[slot(u)] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();
  const int dt = blockIdx.y >> 2, rg0 = 2 * (blockIdx.y & 3);  // 256-row tile of W^T, first row group
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int u = i * 256 + tid;
    const int ks = blockIdx.x * 16 + (u >> 7);
    if (ks >= ks_v) continue;
    const int64_t frag = ((int64_t)dt * ks_v + ks) * kFB + rg0 + ((u >> 6) & 1);
    *reinterpret_cast<uint4*>(WTf + frag * 1024 + (u & 63) * 16) = img[slot(u)];
  }
}

// The kept logits of a chunk (d = z - m_tile, fp16, fragment-major) turned into the
// probabilities in place: P' = exp(d + m_tile - lse) (times 1 - v^2, v = z / zscale, with a
// softcap), bf16 rounded to nearest even; rows past the chunk's tokens become 0.  One
// thread per 16-byte unit (8 consecutive vocabulary entries of one token, one tile).
// ks_count: the k steps the logits GEMM wrote; ks_stride: k steps per row of P; lo_ks > 0: also write
// the lo halves (what the bf16 rounding dropped) from that k step on.
__global__ __launch_bounds__(256) void probs_from_kept_kernel(uint4* __restrict__ P, int64_t units, int rows,
                                                              int ks_count, int ks_stride, int lo_ks,
                                                              const float* __restrict__ pm,
                                                              int ntiles, const float* __restrict__ lse_c,
                                                              LogitMap lm) {
  const int64_t uu = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (uu >= units) return;
  const int l = (int)(uu & 63);
  const int64_t fr = uu >> 6;
  const int fb = (int)(fr % kFB);
  const int64_t rest = fr / kFB;
  const int kstep = (int)(rest % ks_count);
  const int tb = (int)(rest / ks_count);
  const int64_t u = (((int64_t)tb * ks_stride + kstep) * kFB + fb) * 64 + l;
  const int tok = tb * kTB + fb * 32 + (l & 31);
  const int v0 = kstep * 16 + 8 * (l >> 5);
  uint4 out = make_uint4(0u, 0u, 0u, 0u);
  if (tok < rows) {
    const uint4 in = P[u];
    const float m = pm[(int64_t)tok * ntiles + v0 / kTA];
    const float c = m - lse_c[tok];
    float e[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t w = u4get(in, h);
      const float d[2] = {f16_lo(w), f16_hi(w)};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float x = __builtin_amdgcn_exp2f((d[k] + c) * kLog2e);
        if (lm.cap_in > 0.0f) {
          const float v = (d[k] + m) / lm.zscale;
          x = x != 0.0f ? x * (1.0f - v * v) : 0.0f;
        }
        e[2 * h + k] = x;
      }
    }
    out = make_uint4(pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]), pack_bf16(e[6], e[7]));
    if (lo_ks > 0) {
      float r[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t w = u4get(out, h);
        r[2 * h] = e[2 * h] - bf16_lo(w);
        r[2 * h + 1] = e[2 * h + 1] - bf16_hi(w);
      }
      P[u + (int64_t)lo_ks * kFB * 64] =
          make_uint4(pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]), pack_bf16(r[4], r[5]), pack_bf16(r[6], r[7]));
    }
  } else if (lo_ks > 0) {
    P[u + (int64_t)lo_ks * kFB * 64] = out;
  }
  P[u] = out;
}

// Q[t, y_t] = P'[t, y_t] - wyf_t = wyf_t (e^{logp_t} - 1) = wyf_t expm1(z_y - lse), computed in
// fp32 and rounded once: for a confident token (P'_y near 1) the difference keeps its full
// relative precision, where e^{logp} - 1 would cancel.  With hi + lo pairs (lo_ks > 0: fp32
// dH) the lo half gets what the rounding dropped.  One thread per token of the chunk; tokens
// with a target outside [0, V) are left alone (their rows get no weight).
template <typename T>
__global__ __launch_bounds__(256) void onehot_fix_kernel(T* __restrict__ P, int rows, int ks_count, int64_t ldp,
                                                         const int32_t* __restrict__ targets_c,
                                                         const float* __restrict__ zy_c,
                                                         const float* __restrict__ lse_c, int V, LogitMap lm,
                                                         int lo_ks) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= rows) return;
  const int y = targets_c[t];
  if (y < 0 || y >= V) return;
  const float zy = zy_c[t];
  float wyf = 1.0f;
  if (lm.cap_in > 0.0f) {
    const float v = zy / lm.zscale;
    wyf = 1.0f - v * v;
  }
  const float q = wyf * expm1f(zy - lse_c[t]);  // zy - lse is the token's logp, bit for bit
  if constexpr (sizeof(T) == 2) {
    char* dst = reinterpret_cast<char*>(P) + frag_off(t, y, ks_count);
    const uint32_t b = pack_bf16(q, 0.0f) & 0xffffu;
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)b;
    if (lo_ks > 0) {  // hi + lo pairs: the lo half gets what the rounding dropped
      char* dlo = reinterpret_cast<char*>(P) + frag_off(t, lo_ks * 16 + y, ks_count);
      *reinterpret_cast<uint16_t*>(dlo) = (uint16_t)(pack_bf16(q - bf16_lo(b), 0.0f) & 0xffffu);
    }
  } else {
    P[(int64_t)t * ldp + y] = q;
  }
}

// Tokens' operand of the dW GEMM: (-c_t H[t, :])^T of the chunk in the fragment-major
// layout with rows = hidden units and k = tokens: [d / 256][t / 16][(d % 256) / 32][lane]
// [8 tokens], lane = d % 32 + 32 ((t % 16) / 8).  Tokens past the chunk, tokens without a
// gradient and hidden units past D are 0.  One thread per 16-byte unit.
__global__ __launch_bounds__(256) void ht_copy_kernel(const __bf16* __restrict__ Hc, int rows, int D,
                                                      int ks_count, int64_t units, const float* __restrict__ g_c,
                                                      const int32_t* __restrict__ targets_c, int V, float dscale,
                                                      uint4* __restrict__ out) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int l = (int)(u & 63);
  const int64_t fr = u >> 6;
  const int fb = (int)(fr % kFB);
  const int64_t rest = fr / kFB;
  const int kstep = (int)(rest % ks_count);
  const int db = (int)(rest / ks_count);
  const int d = db * kTB + fb * 32 + (l & 31);
  const int t0 = kstep * 16 + 8 * (l >> 5);
  float e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int t = t0 + k;
    float x = 0.0f;
    if (d < D && t < rows) {
      const float gt = g_c[t];
      const int y = targets_c[t];
      if (gt != 0.0f && y >= 0 && y < V) {
        const uint32_t hv = *reinterpret_cast<const uint16_t*>(Hc + (int64_t)t * D + d);
        x = -gt * dscale * __uint_as_float(hv << 16);
      }
    }
    e[k] = x;
  }
  out[u] = make_uint4(pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]), pack_bf16(e[6], e[7]));
}

// One band of the dW GEMM's vocabulary-row operand: Q^T for the band's vocabulary entries
// (rows, from band0) and the slice's tokens (k), in the fragment-major layout
// [vr / 256][t / 16][(vr % 256) / 32][lane][8 tokens] with lane = vr % 32 + 32 ((t % 16) / 8),
// from the slice's fragment-major Q (rows = tokens, k = vocabulary: ks_v k steps of ks_stride;
// with hi + lo probabilities only the hi half is read).  Block
// (tb, g) moves one 256-token tile x 64 vocabulary entries (32 fragments of 1 KB each way)
// through LDS: wave w loads the 8 fragments of vocabulary step 4 g + w (8 KB contiguous, one
// kilobyte per instruction); thread (f, j) transposes the 8 x 8 block j of fragment f in
// registers (its 8 tokens are lanes 8 j .. 8 j + 7); the output fragments go back to LDS and
// out one kilobyte per instruction.  LDS slots rotate within each group of 8 units so that
// every 8-lane group of an access touches 8 distinct 16-byte bank columns.  Vocabulary steps
// past Q's width (ks_v) read as 0; Q's token rows past the slice hold finite values that the
// zero rows of the dW GEMM's tokens' operand cancel.
__device__ __forceinline__ int qt_in_slot(int f, int l) { return f * 64 + 8 * (l >> 3) + (((l & 7) + (l >> 3)) & 7); }
__device__ __forceinline__ int qt_out_slot(int F, int L) {
  return F * 64 + 8 * (L >> 3) + (((L & 7) + (L >> 3) + 2 * (F & 1)) & 7);
}
__global__ __launch_bounds__(256) void qt_band_kernel(const uint4* __restrict__ Q, int ks_v, int ks_stride,
                                                      int tiles_t, int band0, int ks_t, uint4* __restrict__ out) {
  __shared__ uint4 lds[32 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int tb = blockIdx.x % tiles_t;  // token tile
  const int g = blockIdx.x / tiles_t;   // 64-entry vocabulary group of the band
  {
    const int v16 = (band0 >> 4) + 4 * g + w;  // this wave's vocabulary step
    const bool in = v16 < ks_v;
    const uint4* src = Q + ((int64_t)tb * ks_stride + v16) * (kFB * 64) + lane;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      lds[qt_in_slot(8 * w + k, lane)] = in ? src[k * 64] : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  const int f = tid >> 3, j = tid & 7;
  uint4 v[8];  // v[k]: token t0 + k, vocabulary entries v0 .. v0 + 7
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = lds[qt_in_slot(f, 8 * j + k)];
  __syncthreads();
  {
    const int t0 = (f & 7) * 32 + (j & 3) * 8;   // within the token tile
    const int v0 = (f >> 3) * 16 + (j >> 2) * 8;  // within the 64-entry group
    const int F = (v0 >> 5) * 16 + (t0 >> 4);
    const int L0 = (v0 & 31) + 32 * ((t0 >> 3) & 1);
#pragma unroll
    for (int m = 0; m < 8; ++m) {  // vocabulary entry v0 + m for tokens t0 .. t0 + 7
      const int wi = m >> 1;
      const bool hi = m & 1;
      lds[qt_out_slot(F, L0 + m)] =
          make_uint4(halves(u4get(v[0], wi), u4get(v[1], wi), hi), halves(u4get(v[2], wi), u4get(v[3], wi), hi),
                     halves(u4get(v[4], wi), u4get(v[5], wi), hi), halves(u4get(v[6], wi), u4get(v[7], wi), hi));
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int F = 8 * w + k;  // vocabulary row group F / 16 of the 64-entry group, token step F % 16
    const int vr = 64 * g + 32 * (F >> 4);
    out[(((int64_t)(vr >> 8) * ks_t + 16 * tb + (F & 15)) * kFA + ((vr & 255) >> 5)) * 64 + lane] =
        lds[qt_out_slot(F, lane)];
  }
}

// ---------------------------------------------------------------------------- small kernels

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// z[t, y_t] = (H[t] . W[y_t]) / tau, one wave per token, fixed summation order.
template <typename T>
__global__ __launch_bounds__(256) void target_logit_kernel(const T* __restrict__ H, const T* __restrict__ W,
                                                           const int32_t* __restrict__ targets, int ntok,
                                                           int D, int V, LogitMap lm, float* __restrict__ zy) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int y = targets[t];
  if (y < 0 || y >= V) {
    if (lane == 0) zy[t] = __builtin_nanf("");
    return;
  }
  constexpr int VEC = 16 / sizeof(T);
  const T* h = H + (int64_t)t * D;
  const T* w = W + (int64_t)y * D;
  float s = 0.0f;
  for (int c = lane * VEC; c < D; c += 64 * VEC) {
    const uint4 hv = *reinterpret_cast<const uint4*>(h + c);
    const uint4 wv = *reinterpret_cast<const uint4*>(w + c);
    if (sizeof(T) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s = fmaf(bf16_lo(u4get(hv, q)), bf16_lo(u4get(wv, q)), s);
        s = fmaf(bf16_hi(u4get(hv, q)), bf16_hi(u4get(wv, q)), s);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) s = fmaf(__uint_as_float(u4get(hv, q)), __uint_as_float(u4get(wv, q)), s);
    }
  }
  s = wave_sum(s);
  if (lane == 0) zy[t] = lm.zscale * (lm.cap_in > 0.0f ? tanh_fast(lm.cap_in * s) : s);
}

struct MergeArgs {
  const float* pm;
  const float* ps;
  int ntiles;
  int rows;
  int64_t t0;
  const float* zy;      // [T]: target logits (written only for targets in [0, V))
  const int32_t* targets;  // [T]
  int V;
  float* lse;           // [T]
  float* logp;          // [T] or NULL
  int mode;               // 0: log-probs only, 1: GRPO terms, 2: cross-entropy terms
  const float* old_logp;
  const float* ref_logp;  // NULL when beta == 0
  const float* adv;
  const int32_t* seq;
  const uint8_t* mask;    // NULL = all tokens count
  const double* wseq;     // per-sequence token weight
  float eps_lo, eps_hi, beta;
  float* token_loss;      // NULL allowed
  float* g;
  double* wl;
};

// Two (max, sum-exp) pairs as one: M = max, S = S1 e^(M1 - M) + S2 e^(M2 - M) (an empty
// pair has M = -inf and S = 0).  Symmetric in its arguments, bit for bit.
__device__ __forceinline__ void lse_combine(float& M, float& S, float M2, float S2) {
  const float Mn = fmaxf(M, M2);
  S = (M > -INFINITY ? S * expf(M - Mn) : 0.0f) + (M2 > -INFINITY ? S2 * expf(M2 - Mn) : 0.0f);
  M = Mn;
}

// Merge of the vocabulary tiles' (max, sum-exp) partials, stored token-major; then, for
// the loss, the per-token GRPO terms.  One wave per token: lane l folds tiles l, l + 64,
// ... in order into a running pair (one pass over the partials), then the 64 pairs
// combine in a fixed butterfly (both lanes of a step compute the same bits), so the
// result depends on the vocabulary size only, never on the chunking.
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool valid = j < a.rows;
  const float* pm = a.pm + (int64_t)(valid ? j : 0) * a.ntiles;
  const float* ps = a.ps + (int64_t)(valid ? j : 0) * a.ntiles;
  float M = -INFINITY, S = 0.0f;
  if (valid)
    for (int i = lane; i < a.ntiles; i += 64) lse_combine(M, S, pm[i], ps[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float M2 = __shfl_xor(M, m), S2 = __shfl_xor(S, m);
    lse_combine(M, S, M2, S2);
  }
  if (!valid || lane != 0) return;
  const int64_t t = a.t0 + j;
  const float lse = M + logf(S);
  const int y = a.targets[t];
  const float lp = (y >= 0 && y < a.V ? a.zy[t] : __builtin_nanf("")) - lse;
  a.lse[t] = lse;
  if (a.logp) a.logp[t] = lp;
  if (a.mode == 0) return;

  const int s = a.seq[t];
  const bool counted = a.mask == nullptr || a.mask[t] != 0;
  const double w64 = counted ? a.wseq[s] : 0.0;
  const float w = (float)w64;
  float ell, dell;
  if (a.mode == 2) {  // cross-entropy: l = -logp, dl/dlogp = -1 (NaN logp stays NaN in l)
    ell = -lp;
    dell = -1.0f;
  } else if (lp != lp) {  // target outside the vocabulary
    ell = __builtin_nanf("");
    dell = __builtin_nanf("");
  } else {
    const float A = a.adv[s];
    const float rho = expf(lp - a.old_logp[t]);
    const float c = fminf(fmaxf(rho, 1.0f - a.eps_lo), 1.0f + a.eps_hi);
    const float un = rho * A, cl = c * A;
    const float surr = un <= cl ? un : cl;
    const float dsurr = un <= cl ? un : 0.0f;
    float k3 = 0.0f, dk3 = 0.0f;
    if (a.ref_logp) {
      const float d = a.ref_logp[t] - lp;
      const float em1 = expm1f(d);
      k3 = em1 - d;
      dk3 = -em1;
    }
    ell = -(surr - a.beta * k3);
    dell = -dsurr + a.beta * dk3;
  }
  if (a.token_loss) a.token_loss[t] = ell;
  a.g[t] = counted ? w * dell : 0.0f;
  a.wl[t] = w64 != 0.0 ? w64 * (double)ell : 0.0;
}

// x[0, n) = 0 (a kernel rather than a memset, so that the call can be captured in a graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(float* __restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.0f;
}

// Sequence offsets uploaded by value: each launch carries up to 256 of them in its kernel
// arguments, which the runtime copies at launch, so the host array is never read after the
// call returns and no pageable-memory copy (which may synchronize the host) is needed.
constexpr int kCuPerLaunch = 256;
struct CuPiece {
  int32_t v[kCuPerLaunch];
  int32_t first, n;
};
__global__ __launch_bounds__(256) void upload_cu_kernel(const CuPiece piece, int32_t* __restrict__ cu) {
  if ((int)threadIdx.x < piece.n) cu[piece.first + threadIdx.x] = piece.v[threadIdx.x];
}

// cu = {0, T}: the whole stream as one sequence (cross-entropy).
__global__ void whole_stream_cu_kernel(int32_t* cu, int T) {
  if (threadIdx.x == 0) {
    cu[0] = 0;
    cu[1] = T;
  }
}

// Largest s in [0, S) with cu[s] <= t: the sequence of token t.
__device__ __forceinline__ int seq_of(const int32_t* cu, int S, int t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void token_index_kernel(const int32_t* __restrict__ cu, int S, int ntok,
                                                          int chunk, int32_t* __restrict__ seq,
                                                          int32_t* __restrict__ chunk_id,
                                                          int32_t* __restrict__ pos) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= ntok) return;
  const int s = seq_of(cu, S, t);
  seq[t] = s;
  if (chunk_id) chunk_id[t] = t / chunk;
  if (pos) pos[t] = t - cu[s];
}

// Unmasked tokens per sequence; one workgroup per sequence.
__global__ __launch_bounds__(256) void seq_count_kernel(const int32_t* __restrict__ cu,
                                                        const uint8_t* __restrict__ mask,
                                                        int32_t* __restrict__ cnt) {
  __shared__ int part[4];
  const int s = blockIdx.x;
  const int b = cu[s], e = cu[s + 1];
  int n = 0;
  if (mask) {
    for (int t = b + (int)threadIdx.x; t < e; t += 256) n += mask[t] != 0;
  } else if (threadIdx.x == 0) {
    n = e - b;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) cnt[s] = part[0] + part[1] + part[2] + part[3];
}

// Per-sequence token weight: 1 / (S L_i) (sequence mean) or 1 / sum(L) (token mean).
__global__ __launch_bounds__(256) void seq_weight_kernel(const int32_t* __restrict__ cnt, int S, int agg,
                                                         double* __restrict__ wseq) {
  __shared__ long long part[4];
  long long n = 0;
  for (int s = threadIdx.x; s < S; s += 256) n += cnt[s];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = n;
  __syncthreads();
  const long long total = part[0] + part[1] + part[2] + part[3];
  for (int s = threadIdx.x; s < S; s += 256) {
    double w = 0.0;
    if (agg == GRPO_AGG_SEQ_MEAN) {
      if (cnt[s] > 0) w = 1.0 / ((double)S * (double)cnt[s]);
    } else if (total > 0) {
      w = 1.0 / (double)total;
    }
    wseq[s] = w;
  }
}

// loss = sum_t wl[t] in fp64: thread i adds tokens i, i + 1024, ...; then a fixed tree.
__global__ __launch_bounds__(1024) void loss_finalize_kernel(const double* __restrict__ wl, int ntok,
                                                             double* __restrict__ loss) {
  __shared__ double sm[1024];
  double s = 0.0;
  for (int t = threadIdx.x; t < ntok; t += 1024) s += wl[t];
  sm[threadIdx.x] = s;
  for (int stride = 512; stride > 0; stride >>= 1) {
    __syncthreads();
    if ((int)threadIdx.x < stride) sm[threadIdx.x] += sm[threadIdx.x + stride];
  }
  if (threadIdx.x == 0) loss[0] = sm[0];
}

// Fixed-order sum of the split-vocabulary dH partials, then -c_t sum (T: dH's element type).
template <typename T>
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float* __restrict__ part, int ksplit, int rows,
                                                        int D, int V, float dscale,
                                                        const float* __restrict__ g,
                                                        const int32_t* __restrict__ targets, T* __restrict__ dh) {
  const int quads = D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * quads) return;
  const int tok = (int)(idx / quads);
  const int d0 = (int)(idx - (int64_t)tok * quads) * 4;
  const float gt = g[tok];
  const int y = targets[tok];
  float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (gt != 0.0f && y >= 0 && y < V) {
    // all of the token's partials in flight at once, then summed in split order
    float4 pk[kMaxKSplit];
#pragma unroll
    for (int k = 0; k < kMaxKSplit; ++k)
      if (k < ksplit) pk[k] = *reinterpret_cast<const float4*>(part + ((int64_t)k * rows + tok) * D + d0);
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kMaxKSplit; ++k)
      if (k < ksplit) {
        s[0] += pk[k].x; s[1] += pk[k].y; s[2] += pk[k].z; s[3] += pk[k].w;
      }
    const float nc = -gt * dscale;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = nc * s[u];
  }
  store4(dh + (int64_t)tok * D + d0, o[0], o[1], o[2], o[3]);
}

// Group-relative advantages in fp64, one thread per group.
__global__ __launch_bounds__(256) void advantages_kernel(const float* __restrict__ r, int ngroups, int G,
                                                         int std_mode, float eps, float* __restrict__ adv) {
  const int grp = blockIdx.x * 256 + threadIdx.x;
  if (grp >= ngroups) return;
  const float* x = r + (int64_t)grp * G;
  float* o = adv + (int64_t)grp * G;
  bool same = true;
  for (int i = 1; i < G; ++i) same = same && x[i] == x[0];
  if (G == 1 || same) {
    for (int i = 0; i < G; ++i) o[i] = 0.0f;
    return;
  }
  double mu = 0.0;
  for (int i = 0; i < G; ++i) mu += (double)x[i];
  mu /= (double)G;
  double ss = 0.0;
  for (int i = 0; i < G; ++i) {
    const double dv = (double)x[i] - mu;
    ss += dv * dv;
  }
  const double sigma = sqrt(ss / (double)(std_mode == GRPO_STD_UNBIASED ? G - 1 : G));
  for (int i = 0; i < G; ++i) o[i] = (float)(((double)x[i] - mu) / (sigma + (double)eps));
}

// ---------------------------------------------------------------------------- host side

struct Launcher {
  hipStream_t stream;
  grpo_timer* timer;
  template <typename F>
  void run(int kid, F&& f) {
    int slot = -1;
    if (timer) {
      if (timer->used < timer->capacity) slot = timer->used++;
      else ++timer->dropped;
    }
    if (slot >= 0) {
      timer->kid[slot] = kid;
      (void)hipEventRecord(timer->start[slot], stream);
    }
    f();
    if (slot >= 0) (void)hipEventRecord(timer->stop[slot], stream);
  }
};

inline int grid1(int64_t n, int per) { return (int)((n + per - 1) / per); }

// The bf16 kernel that holds this call's tile body (softcap, A layout and split are fixed
// per launch).
template <int KIND>
void (*gemm16_pick(const GemmArgs& g))(const GemmArgs) {
  if constexpr (KIND == KIND_DH || KIND == KIND_DHT) {
    constexpr bool kFrag = KIND == KIND_DHT;
    if (g.ksplit > 1 || g.part_out) {
      if constexpr (kFrag)  // the partials of a banded W^T's later bands are accumulated
        if (g.accumulate) return gemm16_kernel<KIND, true, false, kFrag, false, true>;
      return gemm16_kernel<KIND, true, false, kFrag>;
    }
    return g.dh_f32 ? gemm16_kernel<KIND, false, false, kFrag, true> : gemm16_kernel<KIND, false, false, kFrag>;
  } else if constexpr (KIND == KIND_DW) {
    return gemm16_kernel<KIND, false, false, true>;
  } else {
    const bool cap = g.lm.cap_in > 0.0f;
    if constexpr (KIND == KIND_PROBS) {
      if (g.lo_ks > 0) {  // probabilities as hi + lo pairs (fp32 dH)
        if (g.a_frag)
          return cap ? gemm16_kernel<KIND, false, true, true, true> : gemm16_kernel<KIND, false, false, true, true>;
        return cap ? gemm16_kernel<KIND, false, true, false, true> : gemm16_kernel<KIND, false, false, false, true>;
      }
    }
    if (g.a_frag) return cap ? gemm16_kernel<KIND, false, true, true> : gemm16_kernel<KIND, false, false, true>;
    return cap ? gemm16_kernel<KIND, false, true, false> : gemm16_kernel<KIND, false, false, false>;
  }
}

template <typename T, int KIND>
void launch_gemm(Launcher& L, int kid, const GemmArgs& g) {
  // the largest share of one XCD (the ranges of map_tile differ by at most one tile)
  const int per_xcd = (int)cdiv(g.tiles_a, g.xcd_a) * (int)cdiv(g.tiles_b, 8 / g.xcd_a);
  const int blocks = 8 * per_xcd;
  if constexpr (sizeof(T) == 2) {
    void (*k)(const GemmArgs) = gemm16_pick<KIND>(g);
    L.run(kid, [&] { hipLaunchKernelGGL(k, dim3(blocks), dim3(kThreads), 0, L.stream, g); });
  } else {
    L.run(kid, [&] { hipLaunchKernelGGL((gemm_kernel<T, KIND>), dim3(blocks), dim3(kThreads), 0, L.stream, g); });
  }
}

// Tokens' operand of the bf16 logits GEMMs: the fragment-major copy of the chunk's rows.
inline void enqueue_frag_copy(Launcher& L, const Plan& p, const __bf16* Hc, int rows, char* Hf) {
  L.run(GRPO_K_FRAG_COPY, [&] {
    hipLaunchKernelGGL(frag_copy_kernel, dim3((int)(p.rows_pad / 32), grid1(p.ks_d, 8)), dim3(256), 0, L.stream, Hc,
                       rows, (int)p.D, (int)p.ks_d, Hf);
  });
}

// The plan's fragment-major copies of W, made once per call (bf16): W^T for the dH GEMM
// (else it transposes W tiles in registers) and W for the logits GEMMs (else they read W
// row-major).
template <typename T>
struct WCopies {
  const T* WT = nullptr;
  const char* Wf = nullptr;
  char* WTb = nullptr;   // room for one band of W^T (banded form), else nullptr
  int band_resident = -1;  // the band of W^T now in WTb
  int64_t passes = 0;      // backward passes so far (their parity sets the band order)
};

template <typename T>
WCopies<T> prepare_w(Launcher& L, const Plan& p, const T* W, char* ws) {
  WCopies<T> c;
  if constexpr (sizeof(T) == 2) {
    if (p.T == 0) return c;
    if (p.use_wt) {
      c.WT = reinterpret_cast<const T*>(ws + p.off_WT);
      L.run(GRPO_K_TRANSPOSE_W, [&] {
        hipLaunchKernelGGL(transpose_w_kernel, dim3(grid1(16 * p.ks_v, 256), grid1(cdiv(p.D, kTileA16) * kTileA16, 64)),
                           dim3(256), 0, L.stream, reinterpret_cast<const __bf16*>(W), (int)p.V, (int)p.D,
                           (int)p.ks_v, ws + p.off_WT);
      });
    }
    if (p.wt_bands >= 2) c.WTb = ws + p.off_WTb;
    if (p.use_wf) {
      c.Wf = ws + p.off_Wf;
      L.run(GRPO_K_W_COPY, [&] {
        hipLaunchKernelGGL(frag_copy_kernel, dim3((int)(p.ntiles_v * kTileA16 / 32), grid1(p.ks_d, 8)), dim3(256), 0,
                           L.stream, reinterpret_cast<const __bf16*>(W), (int)p.V, (int)p.D, (int)p.ks_d,
                           ws + p.off_Wf);
      });
    }
  }
  return c;
}

// z[t, y_t] for every token by a row dot product (the fp32 path, and the split backward, which
// runs no logits GEMM).
template <typename T>
void launch_target_logits(Launcher& L, const Plan& p, const T* H, const T* W, const int32_t* targets,
                          const LogitMap& lm, float* zy) {
  if (p.T == 0) return;
  L.run(GRPO_K_TARGET_LOGIT, [&] {
    hipLaunchKernelGGL((target_logit_kernel<T>), dim3(grid1(p.T, 4)), dim3(256), 0, L.stream, H, W, targets,
                       (int)p.T, (int)p.D, (int)p.V, lm, zy);
  });
}

// Arguments shared by the two logits GEMMs of a chunk (W rows x tokens, K = D); Wf is the
// fragment-major copy of W or nullptr.
template <typename T>
GemmArgs logits_args(const Plan& p, const T* W, const char* Wf, const T* Hc, const char* Hf, int rows,
                     const LogitMap& lm) {
  GemmArgs g = {};
  const bool bf16 = sizeof(T) == 2;
  g.a = Wf ? static_cast<const void*>(Wf) : static_cast<const void*>(W);
  g.a_frag = Wf != nullptr;
  g.b = bf16 ? static_cast<const void*>(Hf) : static_cast<const void*>(Hc);
  g.lda = p.D;
  g.ldb = p.D;
  g.a_rows = (int)p.V;
  g.b_rows = rows;
  g.K = (int)p.D;
  g.k_len = (int)p.D;
  g.tiles_a_base = (int)p.ntiles_v;
  g.tiles_a = (int)p.ntiles_v;
  g.tiles_b = (int)cdiv(rows, bf16 ? kTileB16 : kTile);
  g.xcd_a = 8;  // each XCD a share of the vocabulary tiles
  g.group_b = 8;  // B tiles walked together
  g.lm = lm;
  g.V = (int)p.V;
  g.D = (int)p.D;
  g.ksplit = 1;
  g.b_ks = (int)p.ks_d;
  g.p_ks = (int)p.ks_q;
  g.v_ks = (int)(p.dh32 ? p.ks_lo : p.ks_v);  // hi + lo: the hi half's padding k step is written too
  return g;
}

template <typename T>
grpo_status logp_impl(const Plan& p, const grpo_shape* shape, const T* H, const T* W, const int32_t* targets,
                      float* logp, float* lse_out, char* ws, Launcher& L, void* H_host = nullptr,
                      grpo_offload* off = nullptr) {
  const LogitMap lm = make_logit_map(shape);
  if (off) {
    // H to the host on the copy stream, after what `stream` did before this call, beside the GEMMs
    if (hipEventRecord(off->ev_in, L.stream) != hipSuccess ||
        hipStreamWaitEvent(off->copy, off->ev_in, 0) != hipSuccess ||
        hipMemcpyAsync(H_host, H, (size_t)p.T * p.D * sizeof(T), hipMemcpyDeviceToHost, off->copy) != hipSuccess ||
        hipEventRecord(off->ev_done, off->copy) != hipSuccess)
      return GRPO_E_HIP;
  }
  float* zy = reinterpret_cast<float*>(ws + p.off_zy);
  float* lse = lse_out ? lse_out : reinterpret_cast<float*>(ws + p.off_lse);
  float* pm = reinterpret_cast<float*>(ws + p.off_pm);
  float* ps = reinterpret_cast<float*>(ws + p.off_ps);
  char* Hf = ws + p.off_Hf;
  // bf16: the logits GEMM captures the target logits in its epilogue; fp32: a row dot product
  if constexpr (sizeof(T) != 2) launch_target_logits<T>(L, p, H, W, targets, lm, zy);
  const WCopies<T> wc = prepare_w<T>(L, p, W, ws);
  for (int64_t k = 0; k < p.nchunks; ++k) {
    const int64_t t0 = k * p.C;
    const int rows = (int)(p.T - t0 < p.C ? p.T - t0 : p.C);
    if constexpr (sizeof(T) == 2) enqueue_frag_copy(L, p, H + t0 * p.D, rows, Hf);
    GemmArgs g = logits_args<T>(p, W, wc.Wf, H + t0 * p.D, Hf, rows, lm);
    g.pm = pm;
    g.ps = ps;
    if constexpr (sizeof(T) == 2) {
      g.targets = targets + t0;
      g.zy_out = zy + t0;
    }
    launch_gemm<T, KIND_LSE>(L, GRPO_K_LOGITS_LSE, g);
    MergeArgs m = {};
    m.pm = pm;
    m.ps = ps;
    m.ntiles = (int)p.ntiles_v;
    m.rows = rows;
    m.t0 = t0;
    m.zy = zy;
    m.targets = targets;
    m.V = (int)p.V;
    m.lse = lse;
    m.logp = logp;
    L.run(GRPO_K_MERGE, [&] {
      hipLaunchKernelGGL(merge_kernel, dim3(grid1(rows, 4)), dim3(256), 0, L.stream, m);
    });
  }
  if (off && hipStreamWaitEvent(L.stream, off->ev_done, 0) != hipSuccess) return GRPO_E_HIP;
  return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_E_HIP;
}

// Backward of one chunk, over slices of at most p.bwd_rows tokens (the plan's size of the
// probability buffer): the softmax probabilities (recomputed by the PROBS GEMM from the
// forward's log-sum-exp, unless P already holds the whole chunk's), then
// dH = g (z'_y W[y] - P' W) (dH GEMM, split over the vocabulary when the slice is too small
// to fill the GPU) and, if requested, dW (+)= Gx^T H.  Hf holds the chunk's fragment-major
// hidden states (bf16).
// dH_c: [rows, D] of T, or fp32 when the plan writes fp32 dH for bf16 inputs (the
// probabilities then as hi + lo pairs, the dH GEMM's reduction over both halves).
template <typename T>
void backward_chunk(Launcher& L, const Plan& p, const T* W, WCopies<T>& wc, const T* Hc, char* Hf, int rows,
                    int64_t k, const float* lse_c, const float* g_c, const int32_t* targets_c, void* dH_c, T* P,
                    float* part, const LogitMap& lm, const float* zy_c, bool probs_ready, float* dW,
                    char* Qt) {
  const bool bf16 = sizeof(T) == 2;
  const bool out32 = bf16 && p.dh32;
  const int64_t dh_esize = out32 ? 4 : (int64_t)sizeof(T);
  const int srows = (int)(p.bwd_rows > 0 && p.bwd_rows < rows ? p.bwd_rows : rows);
  for (int r0 = 0; r0 < rows; r0 += srows) {
    const int sr = rows - r0 < srows ? rows - r0 : srows;
    const float* lse_s = lse_c + r0;
    const float* g_s = g_c + r0;
    const int32_t* targets_s = targets_c + r0;
    const float* zy_s = zy_c + r0;
    const T* Hs = Hc + (int64_t)r0 * p.D;
    void* dH_s = reinterpret_cast<char*>(dH_c) + (int64_t)r0 * p.D * dh_esize;
    if (!probs_ready) {
      const char* Hf_s = Hf;
      if constexpr (sizeof(T) == 2) {
        // the previous slice's dW operand replaced the chunk's hidden-state copy
        if (dW && r0 > 0) enqueue_frag_copy(L, p, Hc, rows, Hf);
        Hf_s = Hf + (int64_t)(r0 / kTileB16) * p.ks_d * kFB * 1024;
      }
      GemmArgs gp = logits_args<T>(p, W, wc.Wf, Hs, Hf_s, sr, lm);
      gp.lo_ks = out32 ? (int)p.ks_lo : 0;
      gp.lse = lse_s;
      gp.p = P;
      gp.ldp = p.ldp;
      gp.g = g_s;
      gp.targets = targets_s;
      gp.zy = zy_s;
      launch_gemm<T, KIND_PROBS>(L, GRPO_K_PROBS, gp);
    }

    L.run(GRPO_K_ONEHOT_FIX, [&] {
      hipLaunchKernelGGL((onehot_fix_kernel<T>), dim3(grid1(sr, 256)), dim3(256), 0, L.stream, P, sr, (int)p.ks_q,
                         p.ldp, targets_s, zy_s, lse_s, (int)p.V, lm, out32 ? (int)p.ks_lo : 0);
    });

    // dH^T tiles: hidden x tokens, K = vocabulary, split over the vocabulary if needed.  With
    // hi + lo probabilities (fp32 dH) the reduction runs over the hi half (ks_lo k steps, the
    // part past V zero) and then the lo half, W's vocabulary index starting again at 0.
    const int64_t Kd = out32 ? p.ks_lo * 16 + p.V : p.V;
    const int ks_plan = dh_ksplit(sr, p.D, p.V, p.dtype);
    const int k_len = (int)(cdiv(cdiv(Kd, ks_plan), p.bk) * p.bk);
    const int ksplit = (int)cdiv(Kd, k_len);
    GemmArgs gd = {};
    gd.a = wc.WT ? static_cast<const void*>(wc.WT) : static_cast<const void*>(W);
    gd.b = P;
    gd.lda = p.D;
    gd.ldb = p.ldp;
    gd.a_rows = (int)p.D;
    gd.b_rows = sr;
    gd.K = (int)Kd;
    gd.k_len = k_len;
    gd.tiles_a_base = (int)cdiv(p.D, bf16 ? kTileA16 : kTile);
    gd.tiles_a = gd.tiles_a_base * ksplit;
    gd.tiles_b = (int)cdiv(sr, bf16 ? kTileB16 : kTile);
    gd.group_b = bf16 ? 4 : 2;  // 8 W^T tiles x 4 token tiles per XCD round (bf16)
    // XCD grid: each XCD takes at least group_b token tiles where there are enough (a slice of
    // 16 token tiles: 2 x 4 XCDs, 8 hidden x 4 token tiles each), the hidden tiles split over
    // the rest, so the 32 workgroups of an XCD share as many operand rows as they can.
    int xb = 8;
    while (xb > 1 && gd.tiles_b / xb < gd.group_b) xb >>= 1;
    gd.xcd_a = 8 / xb;
    gd.b_ks = (int)p.ks_q;
    gd.a_ks = (int)p.ks_v;
    gd.a_wrap = out32 ? (int)p.ks_lo : 0;
    gd.lm = lm;
    gd.zy = zy_s;
    gd.g = g_s;
    gd.targets = targets_s;
    gd.dh = dH_s;
    gd.dh_f32 = out32;
    gd.part = part;
    gd.V = (int)p.V;
    gd.D = (int)p.D;
    gd.ksplit = ksplit;
    bool reduce = ksplit > 1;
    if constexpr (sizeof(T) == 2) {
      if (wc.WTb) {
        // Banded W^T: band by band of the vocabulary, the band's rows of W transposed into the
        // workspace, then the dH GEMM over the band (split ks_plan ways; a split past the band's
        // end adds zeros), its fp32 partials written by the first band and accumulated by the
        // others.  Consecutive passes walk the bands in opposite orders, so each pass after the
        // first starts on the band that is already in place.
        const int nb = (int)p.wt_bands;
        const bool down = (wc.passes & 1) != 0;
        const int64_t band = p.wt_band_ks * 16;
        const int64_t dpad = cdiv(p.D, kTileA16) * kTileA16;
        gd.a = wc.WTb;
        gd.a_ks = (int)p.wt_band_ks;
        gd.part_out = 1;
        gd.ksplit = ks_plan;
        gd.tiles_a = gd.tiles_a_base * ks_plan;
        for (int i = 0; i < nb; ++i) {
          const int b = down ? nb - 1 - i : i;
          const int64_t v0 = b * band;
          const int64_t vn = p.V - v0 < band ? p.V - v0 : band;
          if (b != wc.band_resident) {
            L.run(GRPO_K_TRANSPOSE_W, [&] {
              hipLaunchKernelGGL(transpose_w_kernel, dim3(grid1(band, 256), grid1(dpad, 64)), dim3(256), 0, L.stream,
                                 reinterpret_cast<const __bf16*>(W) + v0 * p.D, (int)vn, (int)p.D,
                                 (int)p.wt_band_ks, wc.WTb);
            });
            wc.band_resident = b;
          }
          gd.k_base = (int)v0;
          gd.K = (int)(v0 + vn);
          gd.k_len = (int)(cdiv(cdiv(vn, ks_plan), kBK16) * kBK16);
          gd.a_koff = (int)(v0 / 16);
          gd.accumulate = i > 0;
          launch_gemm<T, KIND_DHT>(L, GRPO_K_DH_GEMM, gd);
        }
        reduce = true;
      } else if (wc.WT) {
        launch_gemm<T, KIND_DHT>(L, GRPO_K_DH_GEMM, gd);
      } else {
        launch_gemm<T, KIND_DH>(L, GRPO_K_DH_GEMM, gd);
      }
    } else {
      launch_gemm<T, KIND_DH>(L, GRPO_K_DH_GEMM, gd);
    }
    ++wc.passes;
    if (reduce) {
      const int nsplit = gd.ksplit;
      L.run(GRPO_K_DH_REDUCE, [&] {
        const dim3 grid(grid1((int64_t)sr * (p.D / 4), 256));
        if (out32)
          hipLaunchKernelGGL((dh_reduce_kernel<float>), grid, dim3(256), 0, L.stream, part, nsplit, sr, (int)p.D,
                             (int)p.V, lm.dscale, g_s, targets_s, reinterpret_cast<float*>(dH_s));
        else
          hipLaunchKernelGGL((dh_reduce_kernel<T>), grid, dim3(256), 0, L.stream, part, nsplit, sr, (int)p.D,
                             (int)p.V, lm.dscale, g_s, targets_s, reinterpret_cast<T*>(dH_s));
      });
    }
    if constexpr (sizeof(T) == 2) {
      if (dW) {
        // dW (+)= Gx^T H: the tokens' operand (-c H)^T of the slice replaces the chunk's
        // hidden-state copy (no longer needed once the slice's recompute GEMM has run), then,
        // band by band of the plan's vocabulary tiles, Q^T of the band in fragment-major order
        // and the dW GEMM with the band's vocabulary as rows, the hidden units as columns and
        // the slice's tokens as K.
        const int ks_t = (int)(cdiv(sr, kTileB16) * kTileB16 / 16);
        const int64_t units = cdiv(p.D, kTileB16) * ks_t * kFB * 64;
        L.run(GRPO_K_HT_COPY, [&] {
          hipLaunchKernelGGL(ht_copy_kernel, dim3(grid1(units, 256)), dim3(256), 0, L.stream,
                             reinterpret_cast<const __bf16*>(Hs), sr, (int)p.D, ks_t, units, g_s, targets_s,
                             (int)p.V, lm.dscale, reinterpret_cast<uint4*>(Hf));
        });
        for (int64_t b0 = 0; b0 < p.ntiles_v; b0 += p.qt_tiles) {
          const int nb = (int)(p.ntiles_v - b0 < p.qt_tiles ? p.ntiles_v - b0 : p.qt_tiles);
          const int band0 = (int)(b0 * kTileA16);
          const int tiles_t = ks_t / 16;  // 256-token tiles of the slice
          L.run(GRPO_K_QT_BAND, [&] {
            hipLaunchKernelGGL(qt_band_kernel, dim3(tiles_t * nb * (kTileA16 / 64)), dim3(256), 0, L.stream,
                               reinterpret_cast<const uint4*>(P), (int)p.ks_v, (int)p.ks_q, tiles_t, band0, ks_t,
                               reinterpret_cast<uint4*>(Qt));
          });
          // A: (-c H)^T (rows = hidden units), B: the band of Q^T (rows = vocabulary entries)
          GemmArgs gw = {};
          gw.a = Hf;
          gw.a_frag = 1;
          gw.b = Qt;
          gw.a_rows = (int)p.D;
          gw.b_rows = nb * kTileB16;
          gw.K = sr;
          gw.k_len = sr;
          gw.tiles_a_base = (int)cdiv(p.D, kTileA16);
          gw.tiles_a = gw.tiles_a_base;
          gw.tiles_b = nb;
          gw.xcd_a = nb >= 8 ? 1 : nb >= 4 ? 2 : nb >= 2 ? 4 : 8;  // 8 / xcd_a XCD ranges of the band
          gw.group_b = 4;
          gw.b_ks = ks_t;
          gw.V = (int)p.V - band0;  // the band's rows relative to its first vocabulary entry
          gw.D = (int)p.D;
          gw.ksplit = 1;
          gw.lm = lm;
          gw.dw = dW + (int64_t)band0 * p.D;
          gw.accumulate = k > 0 || r0 > 0;
          launch_gemm<T, KIND_DW>(L, GRPO_K_DW_GEMM, gw);
        }
      }
    }
  }
}

// Loss forward + backward.  mode 1: GRPO objective; mode 2: cross-entropy (prm, old_logp,
// ref_logp and adv unused; one sequence spanning the stream, token-mean weights).
template <typename T>
grpo_status loss_impl(const Plan& p, const grpo_shape* shape, int mode, const grpo_loss_params* prm, const T* H,
                      const T* W, const int32_t* targets, const int32_t* cu_host, const uint8_t* mask,
                      const float* old_logp, const float* ref_logp, const float* adv, double* loss,
                      float* logp, float* token_loss, void* dH, float* dW, char* ws, Launcher& L) {
  const LogitMap lm = make_logit_map(shape);
  float* zy = reinterpret_cast<float*>(ws + p.off_zy);
  float* lse = reinterpret_cast<float*>(ws + p.off_lse);
  float* pm = reinterpret_cast<float*>(ws + p.off_pm);
  float* ps = reinterpret_cast<float*>(ws + p.off_ps);
  float* gbuf = reinterpret_cast<float*>(ws + p.off_g);
  double* wl = reinterpret_cast<double*>(ws + p.off_wl);
  int32_t* seq = reinterpret_cast<int32_t*>(ws + p.off_seq);
  int32_t* cu = reinterpret_cast<int32_t*>(ws + p.off_cu);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + p.off_cnt);
  double* wseq = reinterpret_cast<double*>(ws + p.off_wseq);
  T* P = reinterpret_cast<T*>(ws + p.off_P);
  char* Hf = ws + p.off_Hf;
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  const int64_t dh_esize = p.dh32 ? 4 : (int64_t)sizeof(T);
  const int S = (int)p.S;
  const int agg = mode == 2 ? (int)GRPO_AGG_TOKEN_MEAN : (int)prm->agg;

  if (mode == 2) {
    hipLaunchKernelGGL(whole_stream_cu_kernel, dim3(1), dim3(64), 0, L.stream, cu, (int)p.T);
  } else {
    for (int first = 0; first < S + 1; first += kCuPerLaunch) {
      CuPiece piece;
      piece.first = first;
      piece.n = S + 1 - first < kCuPerLaunch ? S + 1 - first : kCuPerLaunch;
      for (int i = 0; i < piece.n; ++i) piece.v[i] = cu_host[first + i];
      hipLaunchKernelGGL(upload_cu_kernel, dim3(1), dim3(256), 0, L.stream, piece, cu);
    }
  }
  L.run(GRPO_K_TOKEN_INDEX, [&] {
    if (p.T > 0)
      hipLaunchKernelGGL(token_index_kernel, dim3(grid1(p.T, 256)), dim3(256), 0, L.stream, cu, S, (int)p.T,
                         (int)(p.C > 0 ? p.C : 1), seq, (int32_t*)nullptr, (int32_t*)nullptr);
    hipLaunchKernelGGL(seq_count_kernel, dim3(S), dim3(256), 0, L.stream, cu, mask, cnt);
    hipLaunchKernelGGL(seq_weight_kernel, dim3(1), dim3(256), 0, L.stream, cnt, S, agg, wseq);
  });
  // bf16: the logits GEMM captures the target logits in its epilogue; fp32: a row dot product
  if constexpr (sizeof(T) != 2) launch_target_logits<T>(L, p, H, W, targets, lm, zy);
  WCopies<T> wc = prepare_w<T>(L, p, W, ws);
  for (int64_t k = 0; k < p.nchunks; ++k) {
    const int64_t t0 = k * p.C;
    const int rows = (int)(p.T - t0 < p.C ? p.T - t0 : p.C);
    const T* Hc = H + t0 * p.D;
    if constexpr (sizeof(T) == 2) enqueue_frag_copy(L, p, Hc, rows, Hf);
    const bool keep = sizeof(T) == 2 && shape->keep_chunk_logits;
    GemmArgs gl = logits_args<T>(p, W, wc.Wf, Hc, Hf, rows, lm);
    gl.pm = pm;
    gl.ps = ps;
    if constexpr (sizeof(T) == 2) {
      gl.targets = targets + t0;
      gl.zy_out = zy + t0;
    }
    if constexpr (sizeof(T) == 2) {
      if (keep) {
        gl.p = P;
        launch_gemm<T, KIND_LSES>(L, GRPO_K_LOGITS_LSE, gl);
      } else {
        launch_gemm<T, KIND_LSE>(L, GRPO_K_LOGITS_LSE, gl);
      }
    } else {
      launch_gemm<T, KIND_LSE>(L, GRPO_K_LOGITS_LSE, gl);
    }

    MergeArgs m = {};
    m.pm = pm;
    m.ps = ps;
    m.ntiles = (int)p.ntiles_v;
    m.rows = rows;
    m.t0 = t0;
    m.zy = zy;
    m.targets = targets;
    m.V = (int)p.V;
    m.lse = lse;
    m.logp = logp;
    m.mode = mode;
    m.old_logp = old_logp;
    m.ref_logp = ref_logp;
    m.adv = adv;
    m.seq = seq;
    m.mask = mask;
    m.wseq = wseq;
    if (prm) {
      m.eps_lo = prm->clip_eps_low;
      m.eps_hi = prm->clip_eps_high;
      m.beta = prm->beta;
    }
    m.token_loss = token_loss;
    m.g = gbuf;
    m.wl = wl;
    L.run(GRPO_K_MERGE, [&] {
      hipLaunchKernelGGL(merge_kernel, dim3(grid1(rows, 4)), dim3(256), 0, L.stream, m);
    });
    if (keep) {
      const int64_t ks_w = p.dh32 ? p.ks_lo : p.ks_v;  // the k steps the logits GEMM wrote
      const int64_t units = p.rows_pad * ks_w * 2;
      L.run(GRPO_K_PROBS_KEPT, [&] {
        hipLaunchKernelGGL(probs_from_kept_kernel, dim3(grid1(units, 256)), dim3(256), 0, L.stream,
                           reinterpret_cast<uint4*>(P), units, rows, (int)ks_w, (int)p.ks_q,
                           p.dh32 ? (int)p.ks_lo : 0, pm, (int)p.ntiles_v, lse + t0, lm);
      });
    }
    backward_chunk<T>(L, p, W, wc, Hc, Hf, rows, k, lse + t0, gbuf + t0, targets + t0,
                      reinterpret_cast<char*>(dH) + t0 * p.D * dh_esize, P, part, lm, zy + t0, keep, dW,
                      ws + p.off_Qt);
  }
  if (dW && p.nchunks == 0)  // no tokens: the gradient is 0
    hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, L.stream, dW, (int64_t)p.V * p.D);
  L.run(GRPO_K_LOSS_FINALIZE, [&] {
    hipLaunchKernelGGL(loss_finalize_kernel, dim3(1), dim3(1024), 0, L.stream, wl, (int)p.T, loss);
  });
  return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_E_HIP;
}

// Backward of grpo_logp_fwd: dH = (grad / tau) (W[y] - P W) per chunk, from the forward's lse.
// With `off` (p.host_h), H is in pinned host memory: chunk k's rows are copied on the copy
// stream into staging buffer k % 2 of the workspace, after the chunk two before has been used
// from it, and `stream` waits for that copy; so chunk k + 1's copy runs during chunk k's work.
template <typename T>
grpo_status logp_bwd_impl(const Plan& p, const grpo_shape* shape, const T* H, const T* W, const int32_t* targets,
                          const float* lse, const float* grad, void* dH, float* dW, char* ws, Launcher& L,
                          grpo_offload* off = nullptr) {
  const LogitMap lm = make_logit_map(shape);
  T* P = reinterpret_cast<T*>(ws + p.off_P);
  char* Hf = ws + p.off_Hf;
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  float* zy = reinterpret_cast<float*>(ws + p.off_zy);
  const int64_t dh_esize = p.dh32 ? 4 : (int64_t)sizeof(T);
  const bool host = off != nullptr;
  // the target logits: the exact target entry of Q (and the softcap factor there); per chunk
  // from the staged rows when H is on the host
  if (!host) launch_target_logits<T>(L, p, H, W, targets, lm, zy);
  WCopies<T> wc = prepare_w<T>(L, p, W, ws);
  if (host && (hipEventRecord(off->ev_in, L.stream) != hipSuccess ||
               hipStreamWaitEvent(off->copy, off->ev_in, 0) != hipSuccess))
    return GRPO_E_HIP;
  for (int64_t k = 0; k < p.nchunks; ++k) {
    const int64_t t0 = k * p.C;
    const int rows = (int)(p.T - t0 < p.C ? p.T - t0 : p.C);
    const T* Hc = H + t0 * p.D;
    const int b = (int)(k & 1);
    if (host) {
      T* stage = reinterpret_cast<T*>(ws + p.off_Hs + b * p.hs_bytes);
      if ((k >= 2 && hipStreamWaitEvent(off->copy, off->ev_free[b], 0) != hipSuccess) ||
          hipMemcpyAsync(stage, Hc, (size_t)rows * p.D * sizeof(T), hipMemcpyHostToDevice, off->copy) != hipSuccess ||
          hipEventRecord(off->ev_ready[b], off->copy) != hipSuccess ||
          hipStreamWaitEvent(L.stream, off->ev_ready[b], 0) != hipSuccess)
        return GRPO_E_HIP;
      Hc = stage;
      Plan pc = p;  // the chunk's rows only
      pc.T = rows;
      launch_target_logits<T>(L, pc, Hc, W, targets + t0, lm, zy + t0);
    }
    if constexpr (sizeof(T) == 2) enqueue_frag_copy(L, p, Hc, rows, Hf);
    backward_chunk<T>(L, p, W, wc, Hc, Hf, rows, k, lse + t0, grad + t0, targets + t0,
                      reinterpret_cast<char*>(dH) + t0 * p.D * dh_esize, P, part, lm, zy + t0, false, dW,
                      ws + p.off_Qt);
    if (host && hipEventRecord(off->ev_free[b], L.stream) != hipSuccess) return GRPO_E_HIP;
  }
  return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_E_HIP;
}

bool ws_ok(const Plan& p, const void* ws, size_t bytes) {
  if (p.total == 0) return true;
  return ws != nullptr && bytes >= p.total && (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0;
}

// Host-side checks and workspace plan of a grpo_loss_fwd_bwd call (no HIP call).
grpo_status loss_check(const grpo_shape* shape, const grpo_loss_params* params, const void* H, const void* W,
                       const int32_t* targets, const int32_t* cu_seqlens, int64_t num_seqs, const float* old_logp,
                       const float* ref_logp, const float* adv, const double* loss, const void* dH, const float* dW,
                       Plan* p) {
  grpo_status st = validate_shape(shape);
  if (st != GRPO_OK) return st;
  st = validate_loss_params(params);
  if (st != GRPO_OK) return st;
  if (!loss || !adv || !W) return GRPO_E_NULL;
  if (shape->T > 0 && (!H || !targets || !old_logp || !dH)) return GRPO_E_NULL;
  if (params->beta != 0.0f && shape->T > 0 && !ref_logp) return GRPO_E_NULL;
  st = validate_cu(cu_seqlens, num_seqs, shape->T);
  if (st != GRPO_OK) return st;
  if (!aligned16(H) || !aligned16(W) || !aligned16(dH)) return GRPO_E_UNSUPPORTED;
  if (dW && (shape->dtype != GRPO_BF16 || !aligned16(dW))) return GRPO_E_UNSUPPORTED;
  return make_plan(shape, num_seqs, true, p, dW != nullptr);
}

grpo_status loss_run(const Plan& p, const grpo_shape* shape, const grpo_loss_params* params, const void* H,
                     const void* W, const int32_t* targets, const int32_t* cu_seqlens, const uint8_t* mask,
                     const float* old_logp, const float* ref_logp, const float* adv, double* loss, float* logp,
                     float* token_loss, void* dH, float* dW, char* ws, void* stream, grpo_timer* timer) {
  (void)hipGetLastError();
  Launcher L{reinterpret_cast<hipStream_t>(stream), timer};
  const float* ref = params->beta != 0.0f ? ref_logp : nullptr;
  if (p.dtype == GRPO_BF16)
    return loss_impl<__bf16>(p, shape, 1, params, (const __bf16*)H, (const __bf16*)W, targets, cu_seqlens, mask,
                             old_logp, ref, adv, loss, logp, token_loss, dH, dW, ws, L);
  return loss_impl<float>(p, shape, 1, params, (const float*)H, (const float*)W, targets, cu_seqlens, mask,
                          old_logp, ref, adv, loss, logp, token_loss, dH, nullptr, ws, L);
}

// Device address of this device's copy of `scratch`, looked up once per device (with that
// device current) and kept: in host code the array's name is not a device address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
char* g_scratch_ptr[kMaxDevices] = {};

grpo_status static_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GRPO_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GRPO_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GRPO_E_HIP;
    g_scratch_ptr[dev] = reinterpret_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return GRPO_OK;
}

}  // namespace
}  // namespace grpo

using namespace grpo;

extern "C" {

grpo_status grpo_logp_fwd(const grpo_shape* shape, const void* H, const void* W, const int32_t* targets,
                          float* logp, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                          grpo_timer* timer) {
  Plan p;
  grpo_status st = make_plan(shape, 1, false, &p);
  if (st != GRPO_OK) return st;
  if (p.T > 0 && (!H || !W || !targets || !logp)) return GRPO_E_NULL;
  if (!W) return GRPO_E_NULL;
  if (!aligned16(H) || !aligned16(W)) return GRPO_E_UNSUPPORTED;
  if (!ws_ok(p, workspace, workspace_bytes)) return GRPO_E_WORKSPACE;
  if (p.T == 0) return GRPO_OK;
  (void)hipGetLastError();  // clear any stale error so that failures below are this call's
  Launcher L{reinterpret_cast<hipStream_t>(stream), timer};
  char* ws = reinterpret_cast<char*>(workspace);
  if (p.dtype == GRPO_BF16)
    return logp_impl<__bf16>(p, shape, (const __bf16*)H, (const __bf16*)W, targets, logp, lse, ws, L);
  return logp_impl<float>(p, shape, (const float*)H, (const float*)W, targets, logp, lse, ws, L);
}

grpo_status grpo_advantages(const float* rewards, int64_t num_seqs, int64_t group_size, int32_t std_mode,
                            float eps, float* adv, void* stream) {
  if (!rewards || !adv) return GRPO_E_NULL;
  if (num_seqs < 1 || group_size < 1 || num_seqs % group_size != 0 || num_seqs > INT32_MAX) return GRPO_E_SHAPE;
  if (std_mode != GRPO_STD_UNBIASED && std_mode != GRPO_STD_POPULATION) return GRPO_E_VALUE;
  if (!isfinite(eps) || eps < 0.0f) return GRPO_E_VALUE;
  (void)hipGetLastError();
  const int ngroups = (int)(num_seqs / group_size);
  hipLaunchKernelGGL(advantages_kernel, dim3(grid1(ngroups, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), rewards, ngroups, (int)group_size, (int)std_mode, eps,
                     adv);
  return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_E_HIP;
}

grpo_status grpo_loss_fwd_bwd(const grpo_shape* shape, const grpo_loss_params* params, const void* H,
                              const void* W, const int32_t* targets, const int32_t* cu_seqlens, int64_t num_seqs,
                              const uint8_t* mask, const float* old_logp, const float* ref_logp, const float* adv,
                              double* loss, float* logp, float* token_loss, void* dH, float* dW,
                              void* workspace, size_t workspace_bytes, void* stream, grpo_timer* timer) {
  Plan p;
  grpo_status st = loss_check(shape, params, H, W, targets, cu_seqlens, num_seqs, old_logp, ref_logp, adv, loss, dH,
                              dW, &p);
  if (st != GRPO_OK) return st;
  if (!ws_ok(p, workspace, workspace_bytes)) return GRPO_E_WORKSPACE;
  return loss_run(p, shape, params, H, W, targets, cu_seqlens, mask, old_logp, ref_logp, adv, loss, logp, token_loss,
                  dH, dW, reinterpret_cast<char*>(workspace), stream, timer);
}

grpo_status grpo_loss_fwd_bwd_static(const grpo_shape* shape, const grpo_loss_params* params, const void* H,
                                     const void* W, const int32_t* targets, const int32_t* cu_seqlens,
                                     int64_t num_seqs, const uint8_t* mask, const float* old_logp,
                                     const float* ref_logp, const float* adv, double* loss, float* logp,
                                     float* token_loss, void* dH, float* dW, void* stream, grpo_timer* timer) {
  Plan p;
  grpo_status st = loss_check(shape, params, H, W, targets, cu_seqlens, num_seqs, old_logp, ref_logp, adv, loss, dH,
                              dW, &p);
  if (st != GRPO_OK) return st;
  if (p.total > kStaticScratchBytes) return GRPO_E_SCRATCH;  // before any HIP call
  char* ws = nullptr;
  st = static_scratch(&ws);
  if (st != GRPO_OK) return st;
  return loss_run(p, shape, params, H, W, targets, cu_seqlens, mask, old_logp, ref_logp, adv, loss, logp, token_loss,
                  dH, dW, ws, stream, timer);
}

grpo_status grpo_logp_bwd(const grpo_shape* shape, const void* H, const void* W, const int32_t* targets,
                          const float* lse, const float* grad_logp, void* dH, float* dW, void* workspace,
                          size_t workspace_bytes, void* stream, grpo_timer* timer) {
  Plan p;
  grpo_status st = make_plan(shape, 1, true, &p, dW != nullptr);
  if (st != GRPO_OK) return st;
  if (!W) return GRPO_E_NULL;
  if (p.T > 0 && (!H || !targets || !lse || !grad_logp || !dH)) return GRPO_E_NULL;
  if (!aligned16(H) || !aligned16(W) || !aligned16(dH)) return GRPO_E_UNSUPPORTED;
  if (dW && (shape->dtype != GRPO_BF16 || !aligned16(dW))) return GRPO_E_UNSUPPORTED;
  if (!ws_ok(p, workspace, workspace_bytes)) return GRPO_E_WORKSPACE;
  if (p.T == 0 && !dW) return GRPO_OK;  // nothing to do
  (void)hipGetLastError();
  Launcher L{reinterpret_cast<hipStream_t>(stream), timer};
  if (p.T == 0) {  // no tokens: dH is empty and the gradient of W is 0
    hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, L.stream, dW, (int64_t)p.V * p.D);
    return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_E_HIP;
  }
  char* ws = reinterpret_cast<char*>(workspace);
  if (p.dtype == GRPO_BF16)
    return logp_bwd_impl<__bf16>(p, shape, (const __bf16*)H, (const __bf16*)W, targets, lse, grad_logp,
                                 dH, dW, ws, L);
  return logp_bwd_impl<float>(p, shape, (const float*)H, (const float*)W, targets, lse, grad_logp, dH,
                              nullptr, ws, L);
}

grpo_status grpo_offload_create(grpo_offload** out) {
  if (!out) return GRPO_E_NULL;
  grpo_offload* o = new grpo_offload();
  bool ok = hipStreamCreateWithFlags(&o->copy, hipStreamNonBlocking) == hipSuccess;
  for (hipEvent_t* e : {&o->ev_in, &o->ev_done, &o->ev_ready[0], &o->ev_ready[1], &o->ev_free[0], &o->ev_free[1]})
    ok = ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    grpo_offload_destroy(o);
    return GRPO_E_HIP;
  }
  *out = o;
  return GRPO_OK;
}

grpo_status grpo_offload_destroy(grpo_offload* o) {
  if (!o) return GRPO_E_NULL;
  if (o->copy) (void)hipStreamSynchronize(o->copy);
  for (hipEvent_t e : {o->ev_in, o->ev_done, o->ev_ready[0], o->ev_ready[1], o->ev_free[0], o->ev_free[1]})
    if (e) (void)hipEventDestroy(e);
  if (o->copy) (void)hipStreamDestroy(o->copy);
  delete o;
  return GRPO_OK;
}

}  // extern "C"

namespace {

// [T, D] elements of `esize` bytes at p, all in pinned (page-locked) host memory
bool pinned_host(const void* p, int64_t T, int64_t D, int esize) {
  if (!p) return false;
  const char* first = static_cast<const char*>(p);
  const char* last = first + (T * D * esize > 0 ? T * D * esize - 1 : 0);
  for (const char* q : {first, last}) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, q) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    if (a.type != hipMemoryTypeHost) return false;
  }
  return true;
}

}  // namespace

extern "C" {

grpo_status grpo_logp_fwd_offload(const grpo_shape* shape, const void* H, const void* W, const int32_t* targets,
                                  float* logp, float* lse, void* H_host, void* workspace, size_t workspace_bytes,
                                  void* stream, grpo_timer* timer, grpo_offload* offload) {
  Plan p;
  grpo_status st = make_plan(shape, 1, false, &p);
  if (st != GRPO_OK) return st;
  if (!W || !offload) return GRPO_E_NULL;
  if (p.T > 0 && (!H || !targets || !logp || !H_host)) return GRPO_E_NULL;
  if (!aligned16(H) || !aligned16(W)) return GRPO_E_UNSUPPORTED;
  if (!ws_ok(p, workspace, workspace_bytes)) return GRPO_E_WORKSPACE;
  if (p.T == 0) return GRPO_OK;
  if (!pinned_host(H_host, p.T, p.D, p.esize)) return GRPO_E_VALUE;
  (void)hipGetLastError();
  Launcher L{reinterpret_cast<hipStream_t>(stream), timer};
  char* ws = reinterpret_cast<char*>(workspace);
  if (p.dtype == GRPO_BF16)
    return logp_impl<__bf16>(p, shape, (const __bf16*)H, (const __bf16*)W, targets, logp, lse, ws, L, H_host,
                             offload);
  return logp_impl<float>(p, shape, (const float*)H, (const float*)W, targets, logp, lse, ws, L, H_host, offload);
}

grpo_status grpo_logp_bwd_offload(const grpo_shape* shape, const void* H_host, const void* W,
                                  const int32_t* targets, const float* lse, const float* grad_logp, void* dH,
                                  float* dW, void* workspace, size_t workspace_bytes, void* stream,
                                  grpo_timer* timer, grpo_offload* offload) {
  Plan p;
  grpo_status st = make_plan(shape, 1, true, &p, dW != nullptr, true);
  if (st != GRPO_OK) return st;
  if (!W || !offload) return GRPO_E_NULL;
  if (p.T > 0 && (!H_host || !targets || !lse || !grad_logp || !dH)) return GRPO_E_NULL;
  if (!aligned16(H_host) || !aligned16(W) || !aligned16(dH)) return GRPO_E_UNSUPPORTED;
  if (dW && (shape->dtype != GRPO_BF16 || !aligned16(dW))) return GRPO_E_UNSUPPORTED;
  if (!ws_ok(p, workspace, workspace_bytes)) return GRPO_E_WORKSPACE;
  if (p.T == 0 && !dW) return GRPO_OK;
  if (p.T > 0 && !pinned_host(H_host, p.T, p.D, p.esize)) return GRPO_E_VALUE;
  (void)hipGetLastError();
  Launcher L{reinterpret_cast<hipStream_t>(stream), timer};
  if (p.T == 0) {  // no tokens: the gradient of W is 0
    hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, L.stream, dW, (int64_t)p.V * p.D);
    return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_E_HIP;
  }
  char* ws = reinterpret_cast<char*>(workspace);
  if (p.dtype == GRPO_BF16)
    return logp_bwd_impl<__bf16>(p, shape, (const __bf16*)H_host, (const __bf16*)W, targets, lse, grad_logp, dH,
                                 dW, ws, L, offload);
  return logp_bwd_impl<float>(p, shape, (const float*)H_host, (const float*)W, targets, lse, grad_logp, dH,
                              nullptr, ws, L, offload);
}

grpo_status grpo_ce_loss_fwd_bwd(const grpo_shape* shape, const void* H, const void* W, const int32_t* targets,
                                 const uint8_t* mask, double* loss, float* logp, float* token_loss, void* dH,
                                 float* dW, void* workspace, size_t workspace_bytes, void* stream,
                                 grpo_timer* timer) {
  Plan p;
  grpo_status st = make_plan(shape, 1, true, &p, dW != nullptr);
  if (st != GRPO_OK) return st;
  if (!loss || !W) return GRPO_E_NULL;
  if (p.T > 0 && (!H || !targets || !dH)) return GRPO_E_NULL;
  if (!aligned16(H) || !aligned16(W) || !aligned16(dH)) return GRPO_E_UNSUPPORTED;
  if (dW && (shape->dtype != GRPO_BF16 || !aligned16(dW))) return GRPO_E_UNSUPPORTED;
  if (!ws_ok(p, workspace, workspace_bytes)) return GRPO_E_WORKSPACE;
  (void)hipGetLastError();
  Launcher L{reinterpret_cast<hipStream_t>(stream), timer};
  char* ws = reinterpret_cast<char*>(workspace);
  // one sequence spanning the stream (its bounds are written on the device): token-mean weights
  if (p.dtype == GRPO_BF16)
    return loss_impl<__bf16>(p, shape, 2, nullptr, (const __bf16*)H, (const __bf16*)W, targets, nullptr, mask,
                             nullptr, nullptr, nullptr, loss, logp, token_loss, dH, dW, ws, L);
  return loss_impl<float>(p, shape, 2, nullptr, (const float*)H, (const float*)W, targets, nullptr, mask, nullptr,
                          nullptr, nullptr, loss, logp, token_loss, dH, nullptr, ws, L);
}

grpo_status grpo_debug_token_index(const int32_t* cu_seqlens, int64_t num_seqs, int64_t T, int64_t chunk_tokens,
                                   int32_t* seq_id, int32_t* chunk_id, int32_t* pos, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (T < 0 || T > INT32_MAX || chunk_tokens < 1) return GRPO_E_SHAPE;
  grpo_status st = validate_cu(cu_seqlens, num_seqs, T);
  if (st != GRPO_OK) return st;
  if (T > 0 && (!seq_id || !chunk_id || !pos)) return GRPO_E_NULL;
  const size_t need = align_up((size_t)(num_seqs + 1) * 4);
  if (!workspace || workspace_bytes < need) return GRPO_E_WORKSPACE;
  if (T == 0) return GRPO_OK;
  (void)hipGetLastError();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* cu = reinterpret_cast<int32_t*>(workspace);
  for (int64_t first = 0; first < num_seqs + 1; first += kCuPerLaunch) {
    CuPiece piece;
    piece.first = (int32_t)first;
    piece.n = (int32_t)(num_seqs + 1 - first < kCuPerLaunch ? num_seqs + 1 - first : kCuPerLaunch);
    for (int i = 0; i < piece.n; ++i) piece.v[i] = cu_seqlens[first + i];
    hipLaunchKernelGGL(upload_cu_kernel, dim3(1), dim3(256), 0, s, piece, cu);
  }
  hipLaunchKernelGGL(token_index_kernel, dim3(grid1(T, 256)), dim3(256), 0, s, cu, (int)num_seqs, (int)T,
                     (int)(chunk_tokens > INT32_MAX ? INT32_MAX : chunk_tokens), seq_id, chunk_id, pos);
  return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_E_HIP;
}

grpo_status grpo_timer_create(int32_t capacity, grpo_timer** out) {
  if (!out) return GRPO_E_NULL;
  if (capacity < 1 || capacity > (1 << 20)) return GRPO_E_VALUE;
  grpo_timer* t = new grpo_timer();
  t->capacity = capacity;
  t->start.resize(capacity);
  t->stop.resize(capacity);
  t->kid.resize(capacity);
  for (int32_t i = 0; i < capacity; ++i) {
    if (hipEventCreate(&t->start[i]) != hipSuccess || hipEventCreate(&t->stop[i]) != hipSuccess) {
      t->capacity = i;  // destroy what was created
      grpo_timer_destroy(t);
      return GRPO_E_HIP;
    }
  }
  *out = t;
  return GRPO_OK;
}

grpo_status grpo_timer_destroy(grpo_timer* t) {
  if (!t) return GRPO_E_NULL;
  for (int32_t i = 0; i < t->capacity; ++i) {
    if (t->start[i]) (void)hipEventDestroy(t->start[i]);
    if (t->stop[i]) (void)hipEventDestroy(t->stop[i]);
  }
  delete t;
  return GRPO_OK;
}

grpo_status grpo_timer_reset(grpo_timer* t) {
  if (!t) return GRPO_E_NULL;
  t->used = 0;
  t->dropped = 0;
  return GRPO_OK;
}

grpo_status grpo_timer_read(grpo_timer* t, int32_t kernel_id, double* total_ms, int64_t* launches,
                            int64_t* dropped) {
  if (!t || !total_ms || !launches) return GRPO_E_NULL;
  if (kernel_id < 0 || kernel_id >= GRPO_K_COUNT) return GRPO_E_VALUE;
  double ms = 0.0;
  int64_t n = 0;
  for (int32_t i = 0; i < t->used; ++i) {
    if (t->kid[i] != kernel_id) continue;
    if (hipEventSynchronize(t->stop[i]) != hipSuccess) return GRPO_E_HIP;
    float e = 0.0f;
    if (hipEventElapsedTime(&e, t->start[i], t->stop[i]) != hipSuccess) return GRPO_E_HIP;
    ms += e;
    ++n;
  }
  *total_ms = ms;
  *launches = n;
  if (dropped) *dropped = t->dropped;
  return GRPO_OK;
}

}  // extern "C"
