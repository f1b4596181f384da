// Scores and fused decode attention: workspace layout and the dispatch of the plain (MSE-key)
// kernels; the kernels themselves are in attention_impl.h, the QJL-key dispatch in
// attention_qjl.hip.
#include "attention_impl.h"

namespace tq {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

AttnLayout attn_workspace_layout(const tq_attn_params* p, int d, int num_cu) {
  AttnLayout L;
  int splits = p->num_splits;
  if (splits <= 0) {
    int64_t pairs = (int64_t)p->batch * p->num_kv_heads;
    if (pairs < 1) pairs = 1;
    int64_t nblk = ((int64_t)p->max_seq_len + 31) / 32;
    if (nblk < 1) nblk = 1;
    // one full round of resident waves (waves per SIMD x 4 SIMDs x CUs): a partial last round
    // would run the chip at a fraction of its occupancy, and every extra wave pays the
    // prologue (operand tables, query operands) and one more partial for the merge; at least
    // 4 blocks of 32 tokens per wave. The round is counted for 2-bit values (other value widths
    // run a fraction of a round more or less).
    const int wpe = attn_wpe(d, p->cb_k->cb.bits, 2, p->qjl_k != nullptr, p->block_table != nullptr);
    const int64_t target = (int64_t)wpe * 4 * num_cu;
    int64_t s_eff = (target + pairs - 1) / pairs;
    const int64_t cap = nblk >= 8 ? nblk / 4 : 1;
    if (s_eff > cap) s_eff = cap;
    if (s_eff < 1) s_eff = 1;
    splits = (int)((s_eff + kAttnWaves - 1) / kAttnWaves);
  }
  L.splits = splits;
  L.qrot_off = 0;
  const size_t qvec = align256((size_t)p->batch * p->num_q_heads * d * sizeof(float));
  // QJL keys also need the sketched queries S q
  const size_t qbytes = p->qjl_k ? 2 * qvec : qvec;
  L.qsk_off = qvec;
  L.part_off = qbytes;
  // one partial per split, plus one for the recent-token window
  const size_t nparts = (size_t)kAttnWaves * splits + (p->window > 0 ? 1 : 0);
  L.total = qbytes + align256(nparts * p->batch * p->num_q_heads * (d + 2) * sizeof(float));
  if (L.total == 0) L.total = 256;
  return L;
}

hipError_t launch_attention(const tq_attn_params* p, const Codebook& ck, const Codebook& cv, const Rotation& rk,
                            const Rotation& rv, float* scores, bool scores_only, const AttnLayout& lay,
                            hipStream_t st) {
  if (p->qjl_k) return launch_attention_qjl(p, ck, cv, rk, rv, scores, scores_only, lay, st);
  switch (rk.d) {
    case 64: return attn_bk<64, false>(p, ck, cv, rk, rv, scores, scores_only, lay, st);
    case 128: return attn_bk<128, false>(p, ck, cv, rk, rv, scores, scores_only, lay, st);
    default: return attn_bk<256, false>(p, ck, cv, rk, rv, scores, scores_only, lay, st);
  }
}

}  // namespace tq
