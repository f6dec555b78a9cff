// K-tail kernels of table row 6 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(6, Fast6)
