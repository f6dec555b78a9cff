// K-tail kernels of table row 0 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(0, Fast0)
