// gemv_bits.hip -- instantiates the GEMV-family launchers for one bit width.
// Built once per supported width with -DQMM_BITS=<b> (2, 3, 4, 5, 6, 8) so the
// template-heavy kernels compile in parallel.
#include "gemv_kernels.h"

#ifndef QMM_BITS
#error "compile with -DQMM_BITS=<bits>"
#endif

namespace qmm {

template <>
hipError_t launch_gemv_bits<QMM_BITS>(const GemvArgs& a, const GemvShape& sh, hipStream_t st) {
    return sh.unit == 64 ? launch_gemv_unit<QMM_BITS, 64>(a, sh, st)
                         : launch_gemv_unit<QMM_BITS, 32>(a, sh, st);
}

template <>
hipError_t launch_batched_bits<QMM_BITS>(const BatchArgs& a, const GemvShape& sh, hipStream_t st) {
    return sh.unit == 64 ? launch_batched_unit<QMM_BITS, 64>(a, sh, st)
                         : launch_batched_unit<QMM_BITS, 32>(a, sh, st);
}

template <>
hipError_t launch_rows_bits<QMM_BITS>(const RowsArgs& a, const RowsShape& sh, hipStream_t st) {
    return sh.unit == 64 ? launch_rows_unit<QMM_BITS, 64>(a, sh, st)
                         : launch_rows_unit<QMM_BITS, 32>(a, sh, st);
}

}  // namespace qmm
