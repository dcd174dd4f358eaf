// Host-side planning of a fused linear cross-entropy call: tile grid of the
// forward reduction, shape of the backward logit block, workspace layout.
// Pure C++ (no HIP), so it can be unit-tested and sanitised on the host.
#pragma once

#include <cstddef>
#include <cstdint>

namespace fce {

enum class Dtype : int { F32 = 0, BF16 = 1 };
enum class Schedule : int { Auto = 0, Token = 1, Vocab = 2 };
// Recompute: the backward rebuilds each logit block from X and W.
// StoreLogits: the forward keeps a chunk's logits (chunk tokens x all V) in
// the workspace and the backward turns them into dZ in place.
// Filtered: Recompute, with dZ tiles whose softmax values are all below
// 2^-12 (and that hold no label) left out of the gradient products (bf16).
enum class Variant : int { Recompute = 0, StoreLogits = 1, Filtered = 2 };

struct Plan {
  int64_t N = 0, H = 0, V = 0;
  Dtype dtype = Dtype::BF16;
  Variant variant = Variant::Recompute;
  int64_t elem_bytes = 2;

  // forward: token tiles x vocabulary splits, each split walks a range of vocab tiles
  // (StoreLogits: of one token block, the forward runs block by block)
  int64_t fwd_tok_tiles = 0;
  int64_t fwd_voc_tiles = 0;
  int64_t fwd_splits = 0;
  int64_t n_pad = 0;  // fwd_tok_tiles * BN: row pitch of the partials

  // backward logit block: C_N tokens x C_V vocabulary columns
  int64_t tile = 0;  // padding granularity of both block dimensions
  int64_t CN = 0, CV = 0;
  int64_t a = 0, b = 0;  // number of token blocks, vocabulary blocks
  int64_t scratch_rows = 0, ldz = 0;
  // dX product split over its contraction (the vocabulary) when its grid
  // would not fill the CUs: each split writes an fp32 partial [C_N][H]
  int64_t dx_splits = 1;

  // workspace layout (byte offsets, 256-byte aligned)
  size_t off_ctrl = 0, off_flags = 0, off_part = 0, off_blockloss = 0, off_lse = 0,
         off_scratch = 0, off_dxpart = 0, total = 0;
  // fp32: the forward's split row statistics (row max m, log2 of the sum of
  // exp(z - m)) per token, float2 [N]; 0 bytes for bf16
  size_t off_stat = 0, stat_bytes = 0;
  // Filtered: kept flags [tt][vt] (filt_tt x filt_vt bytes per logit block,
  // block ia * b + ib at keep + (ia * b + ib) filt_tt filt_vt) and the
  // kept-block lists of the current block
  int64_t filt_tt = 0, filt_vt = 0;
  size_t off_keep = 0, keep_bytes = 0, off_rowlist = 0, off_rowcnt = 0, off_collist = 0,
         off_colcnt = 0, off_roworder = 0, off_colorder = 0;
  size_t scratch_bytes = 0, partial_bytes = 0, dxpart_bytes = 0;
  // X transposed ([H][ldxt] in the input dtype, zero past N), for the dW
  // product as (dW)^T = X^T dZ: bf16 recompute and store-logits only, 0 bytes
  // otherwise
  int64_t ldxt = 0;
  size_t off_xt = 0, xt_bytes = 0;
  int64_t n_loss_blocks = 0;
  int64_t grad_rmw_bytes = 0;
};

// Layout of the small control block at the start of the workspace.
struct Ctrl {
  int32_t n_valid;
  int32_t n_invalid;
  float scale_fwd;  // 1 / D
  float scale_bwd;  // g / D
};

constexpr int kLossBlock = 256;  // tokens per block of the loss reduction
// Filtered: two uint64 counters (kept tiles, all tiles) inside the control slot
constexpr size_t kOffFilterStats = 64;
static_assert(sizeof(Ctrl) <= kOffFilterStats, "filter counters after the control block");

// How the dW and dX tiles of a logit block of tok_tiles x voc_tiles tiles
// share one grid: the splits of dX over the vocabulary, whether the dX tiles
// (the longer kind) go first, and the modelled time of the grid.
struct GradSchedule {
  int64_t splits;
  bool dx_first;
  double seconds;
};
GradSchedule grad_schedule(Dtype dtype, int64_t H, int64_t tile, int64_t tok_tiles,
                           int64_t voc_tiles);

// Returns false if the arguments are invalid (shapes, chunk, overflow).
bool make_plan(int64_t N, int64_t H, int64_t V, Dtype dtype, int64_t chunk, Schedule sched,
               Plan* out, Variant variant = Variant::Recompute);

}  // namespace fce
