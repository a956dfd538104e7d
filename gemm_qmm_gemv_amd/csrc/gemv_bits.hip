// gemv_bits.hip -- instantiates the GEMV-family launchers for one bit width.
// Built once per supported width with -DQMM_BITS=<b> (2, 3, 4, 5, 6, 8, 16) so the
// template-heavy kernels compile in parallel.
#include "gemv_kernels.h"

#ifndef QMM_BITS
#error "compile with -DQMM_BITS=<bits>"
#endif

namespace qmm {

// fp16 weights are only built with 32-code units.
constexpr bool UNIT64 = QMM_BITS != 16;

template <>
hipError_t launch_gemv_bits<QMM_BITS>(const GemvArgs& a, const GemvShape& sh, hipStream_t st) {
    if constexpr (UNIT64)
        if (sh.unit == 64) return launch_gemv_unit<QMM_BITS, 64>(a, sh, st);
    return sh.unit == 32 ? launch_gemv_unit<QMM_BITS, 32>(a, sh, st) : hipErrorInvalidValue;
}

template <>
hipError_t launch_batched_bits<QMM_BITS>(const BatchArgs& a, const GemvShape& sh, hipStream_t st) {
    if constexpr (UNIT64)
        if (sh.unit == 64) return launch_batched_unit<QMM_BITS, 64>(a, sh, st);
    return sh.unit == 32 ? launch_batched_unit<QMM_BITS, 32>(a, sh, st) : hipErrorInvalidValue;
}

template <>
hipError_t launch_rows_bits<QMM_BITS>(const RowsArgs& a, const RowsShape& sh, hipStream_t st) {
    if constexpr (UNIT64)
        if (sh.unit == 64) return launch_rows_unit<QMM_BITS, 64>(a, sh, st);
    return sh.unit == 32 ? launch_rows_unit<QMM_BITS, 32>(a, sh, st) : hipErrorInvalidValue;
}

template <>
hipError_t launch_glu_bits<QMM_BITS>(const GluArgs& a, const GemvShape& sh, hipStream_t st) {
    if constexpr (UNIT64)
        if (sh.unit == 64) return launch_glu_unit<QMM_BITS, 64>(a, sh, st);
    return sh.unit == 32 ? launch_glu_unit<QMM_BITS, 32>(a, sh, st) : hipErrorInvalidValue;
}

}  // namespace qmm
