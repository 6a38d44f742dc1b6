// k_gemv_q6_k.hip -- the Q6_K GEMV launchers (kernel templates in k_gemv.h).
#include "k_gemv.h"

namespace qgemv {

QGEMV_GEMV_FORMAT_ENTRIES(q6_k, QGEMV_FMT_Q6_K)

}  // namespace qgemv
