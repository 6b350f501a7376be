// Host-side policy of SpecPV's partial-verification buffer ("SpecPV:
// Improving Self-Speculative Decoding for Long-Context Generation via
// Partial Verification", Sec. 3.3 "Rectified with Full Verification";
// App. C and App. D for the buffer size).  Plain host code on host arrays:
// which kind of verification the next step is, and the tree a rectifying
// full verification checks.  The device work of either kind is the existing
// calls (selection, mask, attention, acceptance, commit, summaries).
#include "tv_internal.h"

extern "C" {

int32_t tv_specpv_needs_rectification(int32_t n_partial, int32_t buffer_size) {
  if (n_partial < 0 || buffer_size < 0) return -1;
  // the buffer holds the step's candidates plus at most buffer_size
  // partially verified tokens
  return n_partial > buffer_size ? 1 : 0;
}

tv_status tv_specpv_rectify_tree(const int32_t* buffer_tokens, int32_t n_buffer,
                                 int32_t root_token, const int32_t* parents,
                                 const int32_t* draft_tokens, int32_t n_draft,
                                 int32_t* parents_out, int32_t* tokens_out) {
  if (!buffer_tokens || !parents || !draft_tokens || !parents_out || !tokens_out)
    return TV_ERR_NULL;
  if (n_buffer < 1 || n_draft < 1 || n_buffer + n_draft > TV_MAX_NODES) return TV_ERR_SHAPE;
  if (parents[0] != -1) return TV_ERR_SHAPE;
  for (int32_t j = 1; j < n_draft; ++j)
    if (parents[j] < 0 || parents[j] >= j) return TV_ERR_SHAPE;
  // chain: buffered tokens oldest first, then the current root at node n_buffer
  for (int32_t i = 0; i < n_buffer; ++i) {
    parents_out[i] = i - 1;
    tokens_out[i] = buffer_tokens[i];
  }
  parents_out[n_buffer] = n_buffer - 1;
  tokens_out[n_buffer] = root_token;
  // the draft tree hangs under the current root
  for (int32_t j = 1; j < n_draft; ++j) {
    parents_out[n_buffer + j] = n_buffer + parents[j];
    tokens_out[n_buffer + j] = draft_tokens[j];
  }
  return TV_OK;
}

}  // extern "C"
