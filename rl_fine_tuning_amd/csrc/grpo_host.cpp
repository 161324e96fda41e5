// Host-side argument validation, workspace planning and the chunk schedule of the
// chunked GRPO path.  Nothing here touches the GPU.
//
// Chunking follows "Reinforcement Learning GRPO mit 7x laengerem Kontext" (Unsloth
// docs), section "Chunking der abgeflachten Sequenzlaenge": the batch and context axes
// are flattened into one token stream that is processed a chunk of tokens at a time,
// so the logit memory is that of one chunk (Eq. 3) rather than of the whole stream
// (Eq. 1).  Here a chunk is `chunk_tokens` consecutive tokens of the stream; chunks
// straddle sequence boundaries freely.
#include <math.h>
#include <string.h>

#include "grpo_plan.h"

namespace grpo {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

grpo_status validate_shape(const grpo_shape* s) {
  if (!s) return GRPO_E_NULL;
  if (s->dtype != GRPO_BF16 && s->dtype != GRPO_F32) return GRPO_E_UNSUPPORTED;
  if (s->T < 0 || s->D < 1 || s->V < 1 || s->chunk_tokens < 1) return GRPO_E_SHAPE;
  if (s->T > INT32_MAX || s->V > INT32_MAX || s->chunk_tokens > INT32_MAX) return GRPO_E_SHAPE;
  if (s->D > (1 << 20)) return GRPO_E_SHAPE;
  // 16-byte rows for the vector loads of the GEMMs
  if (s->D % (16 / elem_size(s->dtype)) != 0) return GRPO_E_UNSUPPORTED;
  if (!isfinite(s->temperature) || !(s->temperature > 0.0f)) return GRPO_E_VALUE;
  for (float a : {s->logit_scale_multiply, s->logit_scale_divide, s->logit_softcapping})
    if (!isfinite(a) || a < 0.0f) return GRPO_E_VALUE;
  if (s->keep_chunk_logits != 0 && s->keep_chunk_logits != 1) return GRPO_E_VALUE;
  if (s->keep_chunk_logits && s->dtype != GRPO_BF16) return GRPO_E_UNSUPPORTED;
  const LogitMap m = make_logit_map(s);
  for (float a : {m.zscale, m.dscale, m.cap_in})
    if (!isfinite(a)) return GRPO_E_VALUE;
  if (!(m.zscale > 0.0f) || !(m.dscale > 0.0f)) return GRPO_E_VALUE;
  return GRPO_OK;
}

LogitMap make_logit_map(const grpo_shape* s) {
  const double mul = s->logit_scale_multiply > 0.0f ? s->logit_scale_multiply : 1.0;
  const double div = s->logit_scale_divide > 0.0f ? s->logit_scale_divide : 1.0;
  const double sc = mul / div, tau = s->temperature, cap = s->logit_softcapping;
  LogitMap m;
  m.dscale = (float)(sc / tau);
  if (cap > 0.0) {
    m.zscale = (float)(cap / tau);
    m.cap_in = (float)(sc / cap);
  } else {
    m.zscale = m.dscale;
    m.cap_in = 0.0f;
  }
  return m;
}

grpo_status validate_loss_params(const grpo_loss_params* p) {
  if (!p) return GRPO_E_NULL;
  if (!isfinite(p->clip_eps_low) || !isfinite(p->clip_eps_high) || !isfinite(p->beta))
    return GRPO_E_VALUE;
  if (p->clip_eps_low < 0.0f || p->clip_eps_low >= 1.0f || p->clip_eps_high < 0.0f ||
      p->beta < 0.0f)
    return GRPO_E_VALUE;
  if (p->agg != GRPO_AGG_SEQ_MEAN && p->agg != GRPO_AGG_TOKEN_MEAN) return GRPO_E_VALUE;
  return GRPO_OK;
}

grpo_status validate_cu(const int32_t* cu, int64_t S, int64_t T) {
  if (!cu) return GRPO_E_NULL;
  if (S < 1 || S > INT32_MAX - 1) return GRPO_E_SHAPE;
  if (cu[0] != 0) return GRPO_E_SHAPE;
  for (int64_t i = 0; i < S; ++i)
    if (cu[i + 1] < cu[i]) return GRPO_E_SHAPE;
  if (cu[S] != T) return GRPO_E_SHAPE;
  return GRPO_OK;
}

// Vocabulary split of the dH GEMM for a chunk of `chunk_rows` tokens.  A workgroup
// owns one 256 x 256 tile of dH^T and one workgroup fits a compute unit, so with few
// tiles the reduction over the vocabulary is split and summed afterwards in a fixed
// order.  The cost model counts rounds of workgroups over the compute units per unit
// of split work, plus a small charge per split for the fp32 partials' traffic.
int dh_ksplit(int64_t chunk_rows, int64_t D, int64_t V, int32_t dtype) {
  const int64_t tiles = dtype == GRPO_BF16 ? cdiv(D, kTileA16) * cdiv(chunk_rows, kTileB16)
                                           : cdiv(D, kTile) * cdiv(chunk_rows, kTile);
  const int64_t kblocks = cdiv(V, k_step(dtype));
  int best = 1;
  double best_cost = 1e300;
  for (int k = 1; k <= kMaxKSplit && k <= kblocks; ++k) {
    const double rounds = (double)cdiv(tiles * k, kNumCUs);
    const double cost = rounds / k + 0.02 * k;
    if (cost < best_cost - 1e-12) {
      best_cost = cost;
      best = k;
    }
  }
  return best;
}

grpo_status make_plan(const grpo_shape* s, int64_t S, bool backward, Plan* out) {
  grpo_status st = validate_shape(s);
  if (st != GRPO_OK) return st;
  if (backward && (S < 1 || S > INT32_MAX - 1)) return GRPO_E_SHAPE;
  Plan p;
  p.T = s->T;
  p.D = s->D;
  p.V = s->V;
  p.S = S;
  p.dtype = s->dtype;
  p.esize = elem_size(s->dtype);
  p.bk = k_step(s->dtype);
  p.C = s->T > 0 ? (s->chunk_tokens < s->T ? s->chunk_tokens : s->T) : 0;
  p.nchunks = p.C > 0 ? cdiv(p.T, p.C) : 0;
  const bool bf16 = s->dtype == GRPO_BF16;
  p.ntiles_v = bf16 ? cdiv(p.V, kTileA16) : cdiv(p.V, kTile);
  p.ldp = cdiv(p.V, 16 / p.esize) * (16 / p.esize);
  p.rows_pad = cdiv(p.C, kTileB16) * kTileB16;
  p.ks_d = cdiv(p.D, 16);
  p.ks_v = cdiv(p.V, 16);
  p.backward = backward;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t T = (size_t)p.T, C = (size_t)p.C;
  p.off_zy = take(T * 4);
  p.off_lse = take(T * 4);
  p.off_pm = take((size_t)p.ntiles_v * C * 4);
  p.off_ps = take((size_t)p.ntiles_v * C * 4);
  // the chunk's fragment-major hidden states; in the backward the same region later holds
  // the tokens' operand of the dW GEMM ((D rounded up to 256) x rows_pad bf16)
  if (bf16) {
    size_t hf = (size_t)p.rows_pad * (size_t)p.ks_d * 16 * 2;
    const size_t ht = (size_t)cdiv(p.D, kTileA16) * kTileA16 * (size_t)p.rows_pad * 2;
    if (backward && ht > hf) hf = ht;
    p.off_Hf = take(hf);
  }
  if (backward) {
    p.off_g = take(T * 4);
    p.off_wl = take(T * 8);
    p.off_seq = take(T * 4);
    p.off_cu = take((size_t)(S + 1) * 4);
    p.off_cnt = take((size_t)S * 4);
    p.off_wseq = take((size_t)S * 8);
    p.off_P = bf16 ? take((size_t)p.rows_pad * (size_t)p.ks_v * 16 * 2) : take(C * (size_t)p.ldp * p.esize);
    if (p.nchunks > 0) {
      p.ksplit_full = dh_ksplit(p.C, p.D, p.V, p.dtype);
      const int64_t tail = p.T - (p.nchunks - 1) * p.C;
      p.ksplit_tail = dh_ksplit(tail, p.D, p.V, p.dtype);
    }
    size_t part = 0;
    if (p.ksplit_full > 1) part = (size_t)p.ksplit_full * C * (size_t)p.D * 4;
    const size_t tail_rows = p.nchunks > 0 ? (size_t)(p.T - (p.nchunks - 1) * p.C) : 0;
    if (p.ksplit_tail > 1) {
      const size_t tpart = (size_t)p.ksplit_tail * tail_rows * (size_t)p.D * 4;
      if (tpart > part) part = tpart;
    }
    p.off_part = take(part);
    // A transposed copy of W for the dH GEMM's direct-to-LDS loads, only when the whole
    // workspace still fits in one chunk's fp32 logits.
    p.ldt = cdiv(p.V, 8) * 8;
    const size_t wt = align_up((size_t)p.D * (size_t)p.ldt * 2);
    if (bf16 && p.nchunks > 0 && off + wt <= C * (size_t)p.V * 4) {
      p.use_wt = true;
      p.off_WT = take(wt);
    }
  }
  p.total = off;
  *out = p;
  return GRPO_OK;
}

}  // namespace grpo

extern "C" {

size_t grpo_workspace_bytes(const grpo_shape* shape, int64_t num_seqs, int with_backward) {
  grpo::Plan p;
  if (grpo::make_plan(shape, num_seqs, with_backward != 0, &p) != GRPO_OK) return 0;
  return p.total;
}

const char* grpo_status_string(grpo_status s) {
  switch (s) {
    case GRPO_OK: return "ok";
    case GRPO_E_NULL: return "a required pointer is NULL";
    case GRPO_E_SHAPE: return "a size is out of range or cu_seqlens is inconsistent";
    case GRPO_E_VALUE: return "a scalar argument is out of range or not finite";
    case GRPO_E_WORKSPACE: return "workspace missing, too small or misaligned";
    case GRPO_E_UNSUPPORTED: return "unsupported dtype, alignment or divisibility";
    case GRPO_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* grpo_version(void) { return "grpo-mi355x 0.1 (gfx950)"; }

}  // extern "C"
