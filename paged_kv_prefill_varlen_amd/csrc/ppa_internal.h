// Host-side helpers shared by the validator and the launcher.
#pragma once

#include <cstddef>
#include <cstdint>

#include "ppa.h"

namespace ppa {

// The paged cache reduced to what the address unit needs: a K and a V base
// pointer and, for each, the element strides of (page, kv head, token slot).
// HND vs NHD and split vs combined differ only in these numbers; strides of
// size-1 dimensions are zeroed because they never multiply a non-zero index.
struct CacheView {
  const void* k_base;
  const void* v_base;
  int64_t k_page, k_head, k_tok;
  int64_t v_page, v_head, v_tok;
};

// Fills `view` from validated params (call ppa_validate_shapes first).
void resolve_cache(const ppa_params* p, CacheView* view);

// Bytes of one element of a ppa_dtype (0 for an unknown code).
int dtype_bytes(int32_t dtype);

// snprintf into msg when msg != NULL; returns `status`.
int32_t fail(int32_t status, char* msg, size_t msg_len, const char* fmt, ...);

}  // namespace ppa
