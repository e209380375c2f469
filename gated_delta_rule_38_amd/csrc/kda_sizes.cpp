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

}  // namespace kda
