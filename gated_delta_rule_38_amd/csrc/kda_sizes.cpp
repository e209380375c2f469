// kda_sizes.cpp -- workspace sizes and layouts of the backward calls (host
// code only, shared by the argument checks in kda_api.cpp and the launchers).
#include "kda_launch.h"

namespace kda {

namespace {
constexpr long kChunk = 64;     // tokens per chunk of the chunk form
constexpr long kTokenBlock = 8;  // tokens per checkpoint of the token recurrence

size_t round256(size_t n) { return (n + 255) / 256 * 256; }
}  // namespace

// slots: one per 8 tokens, rounded up, plus one per sequence and a spare, so
// that the first slot of a sequence, cu / 8 + seq, never meets the previous
// sequence's last
size_t backward_workspace_bytes(long tokens_total, int nseq, int H, int dk, int dv) {
    const size_t slots = (size_t)((tokens_total + kTokenBlock - 1) / kTokenBlock + nseq + 1);
    return round256(slots * H * dk * dv * 4);
}

// slots: a sequence from token t0 with n chunks uses t0 / 64 + 2 seq .. + n
size_t bwd_chunk_ckpt_bytes(long tokens_total, int nseq, int H, int dk, int dv) {
    const size_t slots = (size_t)(tokens_total / kChunk) + 2 * (size_t)nseq + 1;
    return round256(slots * H * dk * dv * 4);
}

size_t bwd_chunk_beta_rows(long tokens_total, int H) {
    return ((size_t)tokens_total * H + 63) / 64 * 64;
}

size_t bwd_chunk_workspace_bytes(long tokens_total, int nseq, int H, int dk, int dv) {
    const size_t nk = (size_t)tokens_total * H * dk, nb = bwd_chunk_beta_rows(tokens_total, H);
    return bwd_chunk_ckpt_bytes(tokens_total, nseq, H, dk, dv) +
           (size_t)(dv / 32 - 1) * (3 * nk + nb) * 4;
}

// The two-segment path (chunk_split.hip) pays when the single pass cannot give
// the chip wide slices: eight workgroups per unit (four 32-column slices of the
// first segment, two 64-column slices each of the second segment's transition
// and zero-start parts) must fit the 256 compute units of one MI355X, and the
// sequences must be long enough for the added output pass.  The first segment
// takes 58.3 % of the chunks: with all three parts running, a 32-column chunk
// costs a workgroup about 2.52 us and a 64-column one 3.52 us, so both
// segments then end together.
SplitPlan chunk_split_plan(int B, int T, int H, int dk, int dv) {
    SplitPlan sp;
    const long units = (long)B * H;
    const long nch = (T + kChunk - 1) / kChunk;
    if (dk != 128 || dv != 128 || units <= 0 || units * 8 > 256 || nch < 64) return sp;
    const long c0 = (nch * 583 + 500) / 1000;
    sp.l0 = (int)(c0 * kChunk);
    sp.l1 = T - sp.l0;
    const size_t st = round256((size_t)units * dk * dv * 4);
    sp.off_sm = 0;
    sp.off_phi = st;
    sp.off_r = 2 * st;
    sp.off_z = 3 * st;
    // transition-part outputs: rows seq * T + tau, tau < l1, of dk bf16 per head
    const size_t zrows = (size_t)(B - 1) * T + sp.l1;
    sp.bytes = sp.off_z + round256(zrows * H * dk * 2);
    return sp;
}

}  // namespace kda
