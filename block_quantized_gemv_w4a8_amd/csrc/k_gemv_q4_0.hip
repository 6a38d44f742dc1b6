// k_gemv_q4_0.hip -- the Q4_0 GEMV launchers (kernel templates in k_gemv.h).
#include "k_gemv.h"

namespace qgemv {

QGEMV_GEMV_FORMAT_ENTRIES(q4_0, QGEMV_FMT_Q4_0)

}  // namespace qgemv
