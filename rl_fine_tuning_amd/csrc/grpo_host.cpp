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

#include <initializer_list>

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
  if (s->dh_fp32 != 0 && s->dh_fp32 != 1) return GRPO_E_VALUE;
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

bool decode_ws_mode(int with_backward, bool* backward, bool* dW, bool* host_h) {
  const int base = with_backward & ~GRPO_WS_HOST_H;
  if (base < 0 || base > 2) return false;
  *host_h = (with_backward & GRPO_WS_HOST_H) != 0;
  if (*host_h && base == 0) return false;  // the forward reads H from the device
  *backward = base != 0;
  *dW = base == 2;
  return true;
}

grpo_status make_plan(const grpo_shape* s, int64_t S, bool backward, Plan* out, bool dW, bool host_h) {
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
  // fp32 dH for bf16 inputs: each probability is kept as a bf16 pair hi + lo (lo the rounding
  // residual of hi), in two halves of a row of the probability buffer, so the dH GEMM reads
  // it at about 16 bits of precision; the halves start on a ring stage (32 entries).
  p.dh32 = backward && bf16 && s->dh_fp32 != 0;
  p.ks_lo = p.dh32 ? cdiv(p.ks_v, 2) * 2 : 0;
  p.ks_q = p.dh32 ? 2 * p.ks_lo : p.ks_v;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t T = (size_t)p.T, C = (size_t)p.C;
  // backward from host memory: two buffers of one chunk's rows of H (chunk k + 1 is copied into
  // one while chunk k's GEMMs read the other)
  p.host_h = backward && host_h;
  if (p.host_h && p.nchunks > 0) {
    p.hs_bytes = align_up(C * (size_t)p.D * p.esize);
    p.off_Hs = take(2 * p.hs_bytes);
  }
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
  const size_t bound = C * (size_t)p.V * 4;  // one chunk's fp32 logits
  // Fragment-major copies of W for the bf16 GEMMs: W (rows = vocabulary) for the logits
  // GEMMs and W^T (rows = hidden units) for the dH GEMM.  They make every direct-to-LDS
  // load of the A operand one contiguous kilobyte, and are used when the workspace
  // still fits in one chunk's fp32 logits.
  const size_t wf = bf16 ? align_up((size_t)p.ntiles_v * kTileA16 * (size_t)p.ks_d * 16 * 2) : 0;
  const size_t wt = bf16 ? align_up((size_t)cdiv(p.D, kTileA16) * kTileA16 * (size_t)p.ks_v * 16 * 2) : 0;
  if (!backward) {
    if (bf16 && p.nchunks > 0 && off + wf <= bound) {
      p.use_wf = true;
      p.off_Wf = take(wf);
    }
  } else {
    p.off_g = take(T * 4);
    p.off_wl = take(T * 8);
    p.off_seq = take(T * 4);
    p.off_cu = take((size_t)(S + 1) * 4);
    p.off_cnt = take((size_t)S * 4);
    p.off_wseq = take((size_t)S * 8);

    const int64_t tail = p.nchunks > 0 ? p.T - (p.nchunks - 1) * p.C : 0;
    // dH partials when the backward of a chunk runs over slices of `rows` tokens: the
    // largest over the slices of a full chunk and of the last chunk.
    // (always: the banded W^T form accumulates partials even without a split)
    auto part_bytes = [&](int64_t rows, bool always = false) {
      size_t part = 0;
      for (int64_t n : {p.C, tail}) {
        for (int64_t r0 = 0; r0 < n; r0 += rows) {
          const int64_t sr = n - r0 < rows ? n - r0 : rows;
          const int ks = dh_ksplit(sr, p.D, p.V, p.dtype);
          if ((ks > 1 || always) && (size_t)ks * sr * p.D * 4 > part) part = (size_t)ks * sr * p.D * 4;
        }
      }
      return part;
    };
    auto prob_bytes = [&](int64_t rows) {
      return bf16 ? (size_t)rows * (size_t)p.ks_q * 16 * 2 : C * (size_t)p.ldp * p.esize;
    };
    // Largest layout that fits: both copies with the whole chunk per backward pass; both
    // copies with the backward in two token slices (not with kept logits, which fill the
    // whole chunk's matrix in the forward, nor with dW, whose GEMM would read and write
    // the fp32 [V, D] gradient once more per slice); W^T only; neither.
    const int64_t full = bf16 ? p.rows_pad : (p.C > 0 ? p.C : 1);
    const int64_t half = bf16 ? cdiv(p.rows_pad / kTileB16, 2) * kTileB16 : full;
    const bool keep = s->keep_chunk_logits != 0;
    // With fp32 dH (hi + lo probabilities, twice the buffer) one more layout: the backward in
    // token slices without copies.
    struct Layout { int64_t rows; bool wt, wf; };
    const Layout options[5] = {{full, true, true}, {half, true, true}, {full, true, false}, {full, false, false},
                               {half, false, false}};
    Layout pick = options[3];
    for (const Layout& o : options) {
      if (!bf16 || p.nchunks == 0) break;
      if (&o == &options[4] && !p.dh32) break;
      if (o.rows != full && (keep || dW || o.rows >= full)) continue;
      if (off + align_up(prob_bytes(o.rows)) + align_up(part_bytes(o.rows)) + (o.wt ? wt : 0) + (o.wf ? wf : 0) <=
          bound) {
        pick = o;
        break;
      }
    }
    // Without room for the whole W^T copy (and neither fp32 dH nor dW), the dH GEMM can still
    // read W^T fragment-major: band by band of the vocabulary, each band transposed into the
    // workspace before the GEMM launch that reduces over it, whose fp32 partials accumulate
    // over the bands.  It pays for its transposes (W read and written in each backward pass)
    // from chunks of kBandMinRows tokens on.
    bool bands = false;
    if (bf16 && !pick.wt && !p.dh32 && !dW && p.nchunks > 0 && p.C >= kBandMinRows) {
      const size_t used = off + align_up(prob_bytes(pick.rows)) + align_up(part_bytes(pick.rows, true));
      const size_t ks_bytes = (size_t)cdiv(p.D, kTileA16) * kTileA16 * 16 * 2;  // one k step of the copy
      if (used < bound) {
        const int64_t ks_max = (int64_t)((bound - used) / ks_bytes) / 2 * 2;
        if (ks_max >= kBandMinKs && ks_max < p.ks_v) {
          const int64_t nb = cdiv(p.ks_v, ks_max);
          p.wt_band_ks = cdiv(cdiv(p.ks_v, nb), 2) * 2;
          p.wt_bands = cdiv(p.ks_v, p.wt_band_ks);
          bands = p.wt_bands >= 2;
          if (!bands) p.wt_band_ks = p.wt_bands = 0;
        }
      }
    }
    p.bwd_rows = pick.rows;
    p.off_P = take(prob_bytes(pick.rows));
    p.off_part = take(p.nchunks > 0 ? part_bytes(pick.rows, bands) : 0);
    if (bands) p.off_WTb = take((size_t)cdiv(p.D, kTileA16) * kTileA16 * (size_t)p.wt_band_ks * 16 * 2);
    if (pick.wt) {
      p.use_wt = true;
      p.off_WT = take(wt);
    }
    if (pick.wf) {
      p.use_wf = true;
      p.off_Wf = take(wf);
    }
    // dW: the GEMM's vocabulary-row operand (P' - onehot)^T, fragment-major, one band of
    // vocabulary tiles at a time (32 tiles: two rounds of the GPU's workgroups at D = 4096); a
    // narrower band where 32 would pass the bound, one tile at the least.
    if (bf16 && dW && p.nchunks > 0) {
      const size_t tile_bytes = (size_t)kTileA16 * (size_t)p.rows_pad * 2;
      int64_t nb = 32;
      while (nb > 1 && (nb > p.ntiles_v || off + align_up(nb * tile_bytes) > bound)) nb >>= 1;
      p.qt_tiles = nb;
      p.off_Qt = take(nb * tile_bytes);
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
  bool bwd, dW, host_h;
  if (!grpo::decode_ws_mode(with_backward, &bwd, &dW, &host_h)) return 0;
  if (grpo::make_plan(shape, num_seqs, bwd, &p, dW, host_h) != GRPO_OK) return 0;
  return p.total;
}

grpo_status grpo_plan_info(const grpo_shape* shape, int64_t num_seqs, int with_backward, int64_t info[4]) {
  if (!info) return GRPO_E_NULL;
  grpo::Plan p;
  bool bwd, dW, host_h;
  if (!grpo::decode_ws_mode(with_backward, &bwd, &dW, &host_h)) return GRPO_E_VALUE;
  const grpo_status st = grpo::make_plan(shape, num_seqs, bwd, &p, dW, host_h);
  if (st != GRPO_OK) return st;
  info[0] = p.use_wt ? 1 : p.wt_bands;
  info[1] = p.use_wf ? 1 : 0;
  info[2] = p.bwd_rows;
  info[3] = (int64_t)p.total;
  return GRPO_OK;
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
    case GRPO_E_SCRATCH: return "the call needs more workspace than the static scratch of grpo_loss_fwd_bwd_static";
  }
  return "unknown status";
}

const char* grpo_version(void) { return "grpo-mi355x 0.1 (gfx950)"; }

}  // extern "C"
