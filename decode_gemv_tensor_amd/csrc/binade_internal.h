// Declarations shared by the host and device halves of libbinade.
#ifndef BINADE_INTERNAL_H
#define BINADE_INTERNAL_H

#include <stdint.h>

namespace binade {

// Sum over ranks of count * ((r >> k) + 1): the unary bits of a Rice(k) code.
uint64_t rice_unary_bits(const uint64_t* count_of_rank, uint32_t n, uint32_t k);

// The k in 0..7 with the fewest unary + remainder bits; ties to the smaller k.
uint32_t best_rice_k(const uint64_t* count_of_rank, uint32_t n);

}  // namespace binade

#endif
