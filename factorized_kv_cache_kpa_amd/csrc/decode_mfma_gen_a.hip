// Generic matrix-core decode families with an 8- or 16-wide contracted
// feature dimension (kernel in decode_mfma.hpp): rank caps 2 or 4, up to 32,
// 64 or 128 rows (iG, jG); one query per wave, or two (multi-query decode).
// Families whose registers need more than a quarter of a SIMD's file allow
// four waves per workgroup and one wave per SIMD.
#include "decode_mfma.hpp"

namespace kpa {
namespace mfma {

// arguments: multi-query, QF, rank caps (key, value), row blocks of 32,
// queries per wave, query subgroups, waves per SIMD, waves per workgroup
#define KPA_GEN_QF(QF)                                                                                           \
    KPA_MFMA_GENERIC(false, QF, 2, 2, 1, 1, 1, 2, 8), KPA_MFMA_GENERIC(false, QF, 2, 2, 2, 1, 1, 2, 8),          \
        KPA_MFMA_GENERIC(false, QF, 2, 2, 4, 1, 1, 1, 4), KPA_MFMA_GENERIC(false, QF, 4, 4, 1, 1, 1, 1, 4),      \
        KPA_MFMA_GENERIC(false, QF, 4, 4, 2, 1, 1, 1, 4), KPA_MFMA_GENERIC(false, QF, 4, 4, 4, 1, 1, 1, 4),      \
        KPA_MFMA_GENERIC(true, QF, 2, 2, 1, 2, 1, 1, 4), KPA_MFMA_GENERIC(true, QF, 2, 2, 2, 2, 1, 1, 4),        \
        KPA_MFMA_GENERIC(true, QF, 2, 2, 4, 2, 1, 1, 4), KPA_MFMA_GENERIC(true, QF, 4, 4, 1, 2, 1, 1, 4),        \
        KPA_MFMA_GENERIC(true, QF, 4, 4, 2, 2, 1, 1, 4), KPA_MFMA_GENERIC(true, QF, 4, 4, 4, 2, 1, 1, 4)

const MfmaKernel* generic_kernels_a(int* count) {
    static const MfmaKernel tab[] = {KPA_GEN_QF(8), KPA_GEN_QF(16)};
    *count = (int)(sizeof(tab) / sizeof(tab[0]));
    return tab;
}

}  // namespace mfma
}  // namespace kpa
