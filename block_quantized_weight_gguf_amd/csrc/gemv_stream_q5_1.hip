// The register-staged streaming decode GEMV for Q5_1 (instances of gemv_stream.hpp).
#include "gemv_stream.hpp"

namespace qmm {

template int64_t gemv_stream_fmt<7>(const void*, const void*, const float*, float*, int64_t, int64_t, int, int,
                                     const DecodeEpi&, hipStream_t);

}  // namespace qmm
